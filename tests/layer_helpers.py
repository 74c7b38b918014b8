"""Shared helpers for the GPU tests: run the HIP layer through the C ABI on
seeded inputs and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import oracle
from gpt_causal_self_amd import gpt_attn as ga
from gpt_causal_self_amd.inputs import from_torch, to_torch

# Tolerances.  fp32 inputs: max abs error 1e-4.  bf16 inputs with fp32
# accumulation: |g - r| <= 2e-2 + 1e-2 |r| elementwise, plus a normwise gate
# ||g - r|| / ||r|| <= 1e-2 (the elementwise gate alone is loose next to the
# size of the signal).  Intermediates (q, k, v, merged heads) have tighter
# stage gates: each is one bf16 rounding away from an fp32 accumulation.
TOL = {
    "f32": dict(atol=1e-4, rtol=0.0),
    "bf16": dict(atol=2e-2, rtol=1e-2),
}
NORMWISE_BF16 = 1e-2
STAGE_NORMWISE_BF16 = 5e-3


def device_inputs(inp, device="cuda"):
    d = inp.dtype
    return dict(x=to_torch(inp.x, d, device), W_attn=to_torch(inp.W_attn, d, device),
                b_attn=to_torch(inp.b_attn, d, device), W_proj=to_torch(inp.W_proj, d, device),
                b_proj=to_torch(inp.b_proj, d, device),
                dY=to_torch(inp.dY, d, device) if inp.dY is not None else None)


def gpu_forward(inp, layer=None, save=False, want_ws=False):
    import torch
    B, T, C = inp.x.shape
    own = layer is None
    if own:
        layer = ga.Layer(C, inp.n_head, max(B, 1), max(T, 1), inp.dtype)
    t = device_inputs(inp)
    y = layer.forward(t["x"], t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"],
                      save_for_backward=save)
    torch.cuda.synchronize()
    out = {"y": from_torch(y)}
    if want_ws:
        qkv, o, lse = layer.workspace(B, T)
        out["qkv"] = from_torch(qkv)
        out["o"] = from_torch(o)
        out["lse"] = from_torch(lse)
    if own:
        layer.close()
    return out


def oracle_forward(inp, want=("y",), store_bf16=()):
    """fp64 oracle.  ``store_bf16`` rounds the intermediates that the bf16
    path stores (q/k/v: "qkv", merged heads: "ym") to bf16, isolating a stage's
    own error from the rounding of its bf16 inputs."""
    if inp.dtype != "bf16":
        store_bf16 = ()
    return oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                          inp.n_head, want=want, store_bf16=store_bf16)


def oracle_qkv_headmajor(qkv, H):
    """[B,T,3C] -> [3,B,H,T,hs] (the library's workspace layout)."""
    B, T, C3 = qkv.shape
    C = C3 // 3
    return qkv.reshape(B, T, 3, H, C // H).transpose(2, 0, 3, 1, 4)


def assert_close(g, r, dtype, what="y", normwise=True):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    tol = TOL[dtype]
    err = np.abs(g - r)
    bound = tol["atol"] + tol["rtol"] * np.abs(r)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} / {err.size} elements out of tolerance; worst at {idx}: "
            f"got {g[idx]!r} want {r[idx]!r} (max abs err {err.max():.3e})")
    if dtype == "bf16" and normwise:
        rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
        assert rel <= NORMWISE_BF16, f"{what}: normwise relative error {rel:.3e}"
    return float(err.max())


def assert_qkv_stage(g, r):
    """q/k/v: the GPU rounds an fp32 accumulation of exact products once to
    bf16, the oracle rounds nothing.  bf16 keeps 8 significant bits, so the
    rounding error is at most half an ulp (2^-8 |r|); an fp32 accumulation
    error can move the result across a rounding boundary, giving at most one
    ulp: |g - r| <= 2^-7 |r| (+ 1e-6 for values near zero)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    err = np.abs(g - r)
    bound = 2.0 ** -7 * np.abs(r) + 1e-6
    _report(err, bound, g, r, "q/k/v")


def assert_attention_stage(go, ro, v, elementwise=True):
    """Merged heads o against the oracle fed the bf16-rounded q/k/v.

    The kernel rounds each probability to bf16 before P.V (relative error
    <= 2^-9 per weight) while its normaliser l sums the unrounded fp32
    weights (<= 2^-9 mismatch), a q/k/v element may sit one bf16 ulp (<= 2^-7
    relative) from the oracle's rounding of the exact value, and the output
    is rounded once more (<= 2^-9 |o|).  With M_id = max_{j<=i} |v_jd| (the
    weights sum to 1) this gives |g - r| <= 2^-7 M_id + 2^-8 |r| (+1e-5).
    Always also a normwise gate ||g - r|| / ||r|| <= 5e-3.

    go, ro: [B, T, C]; v: [B, T, C] value block of the oracle's rounded qkv."""
    go = np.asarray(go, np.float64)
    ro = np.asarray(ro, np.float64)
    assert go.shape == ro.shape
    assert np.all(np.isfinite(go))
    rel = np.linalg.norm(go - ro) / max(np.linalg.norm(ro), 1e-30)
    assert rel <= STAGE_NORMWISE_BF16, f"merged heads: normwise relative error {rel:.3e}"
    if elementwise:
        M = np.maximum.accumulate(np.abs(np.asarray(v, np.float64)), axis=1)
        bound = 2.0 ** -7 * M + 2.0 ** -8 * np.abs(ro) + 1e-5
        _report(np.abs(go - ro), bound, go, ro, "merged heads")


def _report(err, bound, g, r, what):
    if not np.all(err <= bound):
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {(err > bound).sum()} elements out of the stage gate; "
                             f"worst at {idx}: got {g[idx]!r} want {r[idx]!r} "
                             f"(bound {bound[idx]:.3e}); max err {err.max():.3e}")
