"""Pins of the oracle's dropout: the Philox4x32-10 generator against its
published known-answer vectors, the drop threshold, the keep rate, p = 0 as
the identity, and the composition (weights dropped after the softmax and
rescaled by 1/(1-p), c_proj output dropped after its bias) against a numpy
assembly of the separately pinned pieces on a tiny case."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from gpt_causal_self_amd.inputs import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(t, 16) for t in line.split()]
        rows.append((w[:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,want", _kat())
def test_philox_known_answers(ctr, key, want):
    assert oracle.philox4x32_10(ctr, key) == want


def test_threshold():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.5) == 1 << 31
    assert oracle.dropout_threshold(0.1) == 429496729          # floor(0.1 * 2^32)
    assert oracle.dropout_threshold(0.9999999999999999) == 0xFFFFFFFF
    assert oracle.dropout_threshold16(0.0) == 0
    assert oracle.dropout_threshold16(0.5) == 1 << 15
    assert oracle.dropout_threshold16(0.1) == 6553                # floor(0.1 * 2^16)
    assert oracle.dropout_threshold16(0.9999999999999999) == 0xFFFF


def test_element_to_counter_mapping():
    """An attention weight (query i, key j) takes the 16-bit half j % 2 of
    word (j % 8) / 2 of Philox({j / 8, i, b*H + h, 1}); a c_proj output element
    (m, n) word n % 4 of Philox({n / 4, m, 0, 2}).  Checked against the
    pinned generator, keys of one group against each other, for a rate at
    which both outcomes are common."""
    p, seed = 0.5, (5 << 32) | 77
    key = [77, 5]
    t16, t32 = oracle.dropout_threshold16(p), oracle.dropout_threshold(p)
    b, h, H = 1, 2, 4
    for i in (0, 3, 9, 130):
        for j in range(0, 24):
            w = oracle.philox4x32_10([j >> 3, i, b * H + h, 1], key)
            u = (w[(j & 7) >> 1] >> (16 * (j & 1))) & 0xFFFF
            assert oracle.dropout_keep_attn(b, h, H, i, j, p, seed) == (u >= t16), (i, j)
    for m in (0, 7, 1025):
        for n in range(0, 12):
            w = oracle.philox4x32_10([n >> 2, m, 0, 2], key)[n & 3]
            assert oracle.dropout_keep_resid(m, n, p, seed) == (w >= t32), (m, n)


def test_keep_rate_and_independence():
    p, seed = 0.3, 1234
    keep = np.array([oracle.dropout_keep_attn(0, 1, 4, i, j, p, seed)
                     for i in range(64) for j in range(64)], dtype=float)
    n = keep.size
    assert abs(keep.mean() - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n)
    res = np.array([oracle.dropout_keep_resid(m, n_, p, seed)
                    for m in range(64) for n_ in range(64)], dtype=float)
    assert abs(res.mean() - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n)
    # the two streams and different seeds give different masks
    assert np.mean(keep != res) > 0.2
    other = np.array([oracle.dropout_keep_attn(0, 1, 4, i, j, p, seed + 1)
                      for i in range(64) for j in range(64)], dtype=float)
    assert np.mean(keep != other) > 0.2


def test_p_zero_is_the_plain_forward():
    inp = make_inputs(2, 19, 32, 4, dtype="f32", seed=3, w_std=0.3, proj_std=0.3)
    a = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 4)["y"]
    b = oracle.forward_dropout(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 4,
                               0.0, 99)["y"]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("p", [0.5, 0.1])
def test_composition_on_a_tiny_case(p):
    B, T, C, H = 2, 6, 8, 2
    hs = C // H
    seed = 77
    inp = make_inputs(B, T, C, H, dtype="f32", seed=11, w_std=0.4, proj_std=0.4,
                      b_attn_std=0.2, b_proj_std=0.2)
    r = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                       want=("P", "qkv"))
    P, qkv = r["P"], r["qkv"]
    ym = np.zeros((B, T, C))
    for b in range(B):
        for h in range(H):
            v = qkv[b, :, 2 * C + h * hs:2 * C + (h + 1) * hs]
            Z = np.array([[oracle.dropout_keep_attn(b, h, H, i, j, p, seed) for j in range(T)]
                          for i in range(T)], dtype=float)
            ym[b, :, h * hs:(h + 1) * hs] = (P[b, h] * Z / (1 - p)) @ v
    y = ym @ inp.W_proj + inp.b_proj
    Z2 = np.array([[oracle.dropout_keep_resid(b * T + t, n, p, seed) for n in range(C)]
                   for b in range(B) for t in range(T)], dtype=float).reshape(B, T, C)
    y = y * Z2 / (1 - p)
    got = oracle.forward_dropout(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                                 p, seed, want_ym=True)
    np.testing.assert_allclose(got["ym"], ym, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["y"], y, rtol=1e-12, atol=1e-14)


def test_backward_p_zero_is_the_plain_backward():
    inp = make_inputs(2, 9, 16, 4, dtype="f32", seed=5, w_std=0.3, proj_std=0.3, with_dY=True)
    a = oracle.backward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, 4)
    b = oracle.backward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, 4,
                        p=1e-300, seed=3)   # keeps every element; scale 1/(1-p) == 1.0
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_backward_with_dropout_matches_finite_differences():
    """L = sum(y * dY) with y the forward with dropout (masks fixed by the
    seed, so L is smooth in every parameter): central differences in fp64
    against the analytic gradient, on sampled entries of every tensor."""
    B, T, C, H = 2, 7, 8, 2
    p, seed = 0.4, 2024
    inp = make_inputs(B, T, C, H, dtype="f32", seed=19, w_std=0.4, proj_std=0.4,
                      b_attn_std=0.2, b_proj_std=0.2, with_dY=True)
    args = {k: np.asarray(getattr(inp, k), np.float64)
            for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    dY = np.asarray(inp.dY, np.float64)

    def loss(a):
        y = oracle.forward_dropout(a["x"], a["W_attn"], a["b_attn"], a["W_proj"], a["b_proj"],
                                   H, p, seed)["y"]
        return float(np.sum(y * dY))

    g = oracle.backward(args["x"], args["W_attn"], args["b_attn"], args["W_proj"],
                        args["b_proj"], dY, H, p=p, seed=seed)
    names = {"x": "dx", "W_attn": "dW_attn", "b_attn": "db_attn", "W_proj": "dW_proj",
             "b_proj": "db_proj"}
    rng = np.random.default_rng(0)
    eps = 1e-6
    for k, gk in names.items():
        flat = args[k].reshape(-1)
        for idx in rng.choice(flat.size, size=min(24, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + eps
            lp = loss(args)
            flat[idx] = old - eps
            lm = loss(args)
            flat[idx] = old
            fd = (lp - lm) / (2 * eps)
            an = g[gk].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (k, idx, fd, an)


def check_single_precision_keep_factor(lib=None):
    """"z32" holds 1/(1-p) as the nearest float.  At p = float32(0.2),
    1/(1-p) = 1.2500000047 whose nearest float is exactly 1.25, so with the
    stored masked gradient ("dyd") db_proj is the column sum of
    bf16(keep * dY * 1.25); at p = 0.5 the factor 2 is exact either way."""
    from test_oracle_pins import _bits_rne_bf16
    B, T, C, H = 1, 9, 16, 2
    inp = make_inputs(B, T, C, H, dtype="bf16", seed=53, w_std=0.3, with_dY=True)
    args = (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, H)
    p = float(np.float32(0.2))
    r = oracle.backward(*args, p=p, seed=5, store_bf16=("dyd", "z32"), lib=lib)
    keep = np.array([[oracle.dropout_keep_resid(m, n, p, 5, lib=lib) for n in range(C)]
                     for m in range(B * T)], dtype=float)
    dyd = _bits_rne_bf16(keep * inp.dY.reshape(-1, C).astype(np.float64) * 1.25)
    np.testing.assert_allclose(r["db_proj"], dyd.sum(0), rtol=1e-13, atol=1e-13)
    r64 = oracle.backward(*args, p=p, seed=5, store_bf16=("dyd",), lib=lib)
    assert not np.array_equal(r64["db_proj"], r["db_proj"])
    a = oracle.backward(*args, p=0.5, seed=5, store_bf16=("dyd", "z32"), lib=lib)
    b = oracle.backward(*args, p=0.5, seed=5, store_bf16=("dyd",), lib=lib)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_single_precision_keep_factor():
    check_single_precision_keep_factor()
