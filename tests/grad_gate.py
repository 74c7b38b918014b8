"""Derived elementwise gate for bf16 gradients.

Every gradient of the layer is a contraction G = sum_r a_r b_r over the
operands the oracle uses (dx: dqkv . W_attn^T; dW_attn: x^T . dqkv;
db_attn: column sums of dqkv; dW_proj: y_m^T . dY; db_proj: column sums of
dY).  On the bf16 path the operands reach the final contraction through a few
bf16 roundings (stored q/k/v, merged heads, their gradients, and the bf16
probabilities / dS fed to the MFMAs), each a zero-mean relative error of at
most 2^-9; over all of them the per-term relative error stays below
eps = 2^-7.  The error of G is then a sum of independent zero-mean terms with
standard deviation at most sigma = eps * sqrt(sum_r a_r^2 b_r^2), and the
gate is the stated bf16 tolerance widened by six such sigmas:
    |g - r| <= 2e-2 + 1e-2 |r| + 6 sigma.
A normwise gate ||g - r|| / ||r|| <= 1e-2 against the exact oracle holds on
top of it.

One correlation is added explicitly.  The columns of the value block of dqkv
sum to the column sums of dO, the stored gradient of the merged heads
(sum_j dv_j = sum_i dO_i sum_j p_ij and every softmax row sums to one), so
the bf16 rounding of each stored dO_i reaches db_attn's value block once per
row with nothing averaging it out: that block's sigma also carries
eps * sqrt(sum_i dO_id^2)."""
from __future__ import annotations

import numpy as np

EPS = 2.0 ** -7
K_SIGMA = 6.0


def sigmas(inp, ref_inter):
    """sigma of each gradient from the oracle's operands (fp64)."""
    B, T, C = inp.x.shape
    x2 = inp.x.reshape(-1, C).astype(np.float64) ** 2
    g2 = ref_inter["dqkv"].reshape(-1, 3 * C) ** 2
    ym2 = ref_inter["ym"].reshape(-1, C) ** 2
    dY2 = inp.dY.reshape(-1, C).astype(np.float64) ** 2
    Wa2 = inp.W_attn.astype(np.float64) ** 2
    db_attn2 = g2.sum(0)
    db_attn2[2 * C:] += (ref_inter["dym"].reshape(-1, C) ** 2).sum(0)
    s = {"dx": np.sqrt(g2 @ Wa2.T).reshape(B, T, C),
         "dW_attn": np.sqrt(x2.T @ g2),
         "db_attn": np.sqrt(db_attn2),
         "dW_proj": np.sqrt(ym2.T @ dY2),
         "db_proj": np.sqrt(dY2.sum(0))}
    return {k: EPS * v for k, v in s.items()}


def check(name, g, r, sigma, normwise=1e-2):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), name
    err = np.abs(g - r)
    bound = 2e-2 + 1e-2 * np.abs(r) + K_SIGMA * sigma
    if not np.all(err <= bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{name}: {(err > bound).sum()} / {err.size} out of the gradient "
                             f"gate; worst at {i}: got {g[i]!r} want {r[i]!r} "
                             f"(bound {bound[i]:.3e}, sigma {sigma[i]:.3e})")
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    assert rel <= normwise, f"{name}: normwise relative error {rel:.3e}"
    return float((err / np.maximum(sigma, 1e-30)).max()), rel
