"""Brute-force causal self-attention in pure Python loops (tiny shapes only).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  A second, independent
rendering of the definition used to pin the C oracle: plain nested loops over
Python floats, one output element at a time, written from page "nanoGPT
global flow", section 2.5 (B) CausalSelfAttention (steps 1-7 of its forward)
and page "nanoGPT architecture explained step by step", section 3, formula
softmax(Q K^T / sqrt(d_k)) V.  The softmax here is computed directly as
exp(s_j) / sum_j' exp(s_j') over the visible keys (no max subtraction), which
is a different route from the oracle's max-shifted two-pass form; on tiny
inputs with moderate scores the two agree to rounding.
"""
from __future__ import annotations

import math


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def forward(x, W_attn, b_attn, W_proj, b_proj, n_head):
    """x [B][T][C] nested lists (or arrays); weights [in][out].
    Returns (y, P) with y [B][T][C] and P [B][H][T][T] as nested lists."""
    x, W_attn, W_proj = _tolist(x), _tolist(W_attn), _tolist(W_proj)
    b_attn = _tolist(b_attn) if b_attn is not None else None
    b_proj = _tolist(b_proj) if b_proj is not None else None
    B, T, C = len(x), len(x[0]), len(x[0][0])
    H = n_head
    hs = C // H

    def c_attn(b, t, n):
        s = b_attn[n] if b_attn is not None else 0.0
        for c in range(C):
            s += x[b][t][c] * W_attn[c][n]
        return s

    qkv = [[[c_attn(b, t, n) for n in range(3 * C)] for t in range(T)]
           for b in range(B)]

    def q(b, h, t, d):
        return qkv[b][t][h * hs + d]

    def k(b, h, t, d):
        return qkv[b][t][C + h * hs + d]

    def v(b, h, t, d):
        return qkv[b][t][2 * C + h * hs + d]

    P = [[[[0.0] * T for _ in range(T)] for _ in range(H)] for _ in range(B)]
    ym = [[[0.0] * C for _ in range(T)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(T):
                e = []
                for j in range(i + 1):
                    s = 0.0
                    for d in range(hs):
                        s += q(b, h, i, d) * k(b, h, j, d)
                    e.append(math.exp(s / math.sqrt(hs)))
                Z = sum(e)
                for j in range(i + 1):
                    P[b][h][i][j] = e[j] / Z
                for d in range(hs):
                    acc = 0.0
                    for j in range(i + 1):
                        acc += P[b][h][i][j] * v(b, h, j, d)
                    ym[b][i][h * hs + d] = acc

    y = [[[0.0] * C for _ in range(T)] for _ in range(B)]
    for b in range(B):
        for t in range(T):
            for n in range(C):
                s = b_proj[n] if b_proj is not None else 0.0
                for c in range(C):
                    s += ym[b][t][c] * W_proj[c][n]
                y[b][t][n] = s
    return y, P
