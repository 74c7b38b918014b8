"""GPU parity of the Block pieces around the attention layer (through the C
ABI, include/gpt_block.h) against the fp64 oracle: LayerNorm, the Pre-LN
attention half-block out = x + attn(ln_1(x)), and the MLP sublayer with its
fused GELU epilogue (with and without the residual add).

Gates.  LayerNorm output and the MLP activations are one bf16 rounding of an
fp32 computation of the exact value: at most one bf16 ulp, |g - r| <= 2^-7 |r|
(+ a small absolute term for values near zero).  Block and MLP outputs are
compared with the oracle that rounds the stored intermediates exactly as the
GPU does (ln_1 output, q/k/v, merged heads; MLP activations), so what remains
is fp32 accumulation order, the bf16 probabilities of P.V and the final
rounding; the tests use projection weights large enough that the sublayer
output is O(1) next to the residual, so its errors are visible through the
final bf16 rounding."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpt_causal_self_amd import gpt_attn as ga
from gpt_causal_self_amd.inputs import (from_torch, make_inputs, make_ln_params,
                                        make_mlp_inputs, to_torch)

pytestmark = pytest.mark.gpu


def _gate(g, r, rel, abs_, what):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - r)
    bound = rel * np.abs(r) + abs_
    if not np.all(err <= bound):
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {(err > bound).sum()} / {err.size} out of the gate; "
                             f"worst at {idx}: got {g[idx]!r} want {r[idx]!r} "
                             f"(bound {bound[idx]:.3e}); max err {err.max():.3e}")


def _ln_gpu(x, w, b):
    import torch
    xt, wt, bt = to_torch(x, "bf16", "cuda"), to_torch(w, "bf16", "cuda"), to_torch(b, "bf16", "cuda")
    out = torch.empty_like(xt)
    ga.gpt_layernorm(xt, wt, bt, out)
    torch.cuda.synchronize()
    return from_torch(out)


@pytest.mark.parametrize("M,C,bias,offset", [
    (300, 256, True, 0.0), (12288, 768, True, 0.0), (37, 1600, False, 0.0), (5, 8, True, 0.0),
    (9, 8192, True, 0.0), (64, 768, True, 40.0), (13, 512, True, 0.0), (301, 768, False, 0.0),
    (7, 1024, True, 0.0)])
def test_layernorm(M, C, bias, offset):
    from gpt_causal_self_amd.inputs import to_dtype
    rng = np.random.default_rng(M + C)
    x = to_dtype(rng.standard_normal((M, C), dtype=np.float32) * 3 + np.float32(offset), "bf16")
    w, b = make_ln_params(C, seed=C, bias=bias)
    g = _ln_gpu(x, w, b)
    r = oracle.layernorm(x, w, b)
    _gate(g, r, 2.0 ** -7, 1e-5, "layernorm")


def test_layernorm_constant_row_gives_the_shift():
    """A constant row has zero variance: the output is exactly b (rstd only
    scales zeros)."""
    from gpt_causal_self_amd.inputs import to_dtype
    C = 768
    x = to_dtype(np.full((4, C), 2.5, np.float32), "bf16")
    w, b = make_ln_params(C, seed=1)
    assert np.array_equal(_ln_gpu(x, w, b), b[None, :].repeat(4, 0))


def _block_inputs(B, T, C, H, bias=True, seed=0, big_proj=True):
    inp = make_inputs(B, T, C, H, bias=bias, dtype="bf16", seed=seed,
                      proj_std=0.2 if big_proj else 0.02 / np.sqrt(24),
                      b_proj_std=0.2 if big_proj else 0.02)
    ln_w, ln_b = make_ln_params(C, seed=seed + 1, bias=bias)
    return inp, ln_w, ln_b


def _block_gpu(inp, ln_w, ln_b, layer=None):
    import torch
    B, T, C = inp.x.shape
    own = layer is None
    if own:
        layer = ga.Layer(C, inp.n_head, B, T, "bf16")
    d = {k: to_torch(getattr(inp, k), "bf16", "cuda")
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    out = torch.empty_like(d["x"])
    ga.gpt_attn_block_forward(layer.h, d["x"], to_torch(ln_w, "bf16", "cuda"),
                              to_torch(ln_b, "bf16", "cuda"), d["W_attn"], d["b_attn"],
                              d["W_proj"], d["b_proj"], inp.n_head, out)
    torch.cuda.synchronize()
    if own:
        layer.close()
    return from_torch(out)


def _block_oracle(inp, ln_w, ln_b):
    return oracle.block_attn_forward(inp.x, ln_w, ln_b, inp.W_attn, inp.b_attn, inp.W_proj,
                                     inp.b_proj, inp.n_head, want_ln=True,
                                     store_bf16=("ln", "qkv", "ym"))


def _block_check(inp, ln_w, ln_b, g):
    r = _block_oracle(inp, ln_w, ln_b)
    y = r["out"] - inp.x.astype(np.float64)
    scale = np.abs(y).max(axis=-1, keepdims=True)
    # one ulp of out, plus the attention stage's own error (probabilities in
    # bf16, <= 2^-8 of the row's largest sublayer output)
    _gate(g, r["out"], 2.0 ** -7, 2.0 ** -8 * scale + 1e-5, "block out")
    rel = np.linalg.norm((g - inp.x) - y) / np.linalg.norm(y)
    assert rel < 1e-2, f"sublayer part normwise error {rel:.3e}"


@pytest.mark.parametrize("B,T,C,H,bias", [(2, 70, 256, 4, True), (1, 129, 128, 4, True),
                                          (3, 64, 256, 8, False), (1, 1, 128, 2, True)])
def test_block_small(B, T, C, H, bias):
    inp, ln_w, ln_b = _block_inputs(B, T, C, H, bias=bias, seed=B * T + C)
    _block_check(inp, ln_w, ln_b, _block_gpu(inp, ln_w, ln_b))


def test_block_ragged_rows_wide_projection():
    """7000 rows at C = 768: the residual c_proj on 96 x 384 tiles, the last
    row tile 88 rows deep."""
    inp, ln_w, ln_b = _block_inputs(7, 1000, 768, 12, seed=17)
    _block_check(inp, ln_w, ln_b, _block_gpu(inp, ln_w, ln_b))


def test_block_gpt2_124m_full():
    """GPT-2 124M shape (B=12, T=1024, C=768, 12 heads), every sequence."""
    inp, ln_w, ln_b = _block_inputs(12, 1024, 768, 12, seed=7)
    _block_check(inp, ln_w, ln_b, _block_gpu(inp, ln_w, ln_b))


def test_block_zero_projection_returns_x_bitwise():
    """W_proj = 0 and b_proj = 0: the sublayer output is exactly zero and the
    residual passes through unrounded."""
    inp, ln_w, ln_b = _block_inputs(2, 96, 256, 4, seed=3)
    inp.W_proj[:] = 0.0
    inp.b_proj[:] = 0.0
    assert np.array_equal(_block_gpu(inp, ln_w, ln_b), inp.x)


def test_block_then_plain_forward_state():
    """The block call clears the saved forward state (a backward after it is
    a STATE error), and the handle still runs a plain forward afterwards."""
    import torch
    inp, ln_w, ln_b = _block_inputs(2, 64, 128, 4, seed=11)
    layer = ga.Layer(128, 4, 2, 64, "bf16")
    d = {k: to_torch(getattr(inp, k), "bf16", "cuda")
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    layer.forward(d["x"], d["W_attn"], d["b_attn"], d["W_proj"], d["b_proj"],
                  save_for_backward=True)
    _block_gpu(inp, ln_w, ln_b, layer=layer)
    with pytest.raises(ga.GptAttnError) as e:
        layer.backward(d["x"], d["W_attn"], d["W_proj"], torch.ones_like(d["x"]))
    assert e.value.code == ga.ERR_STATE
    y = layer.forward(d["x"], d["W_attn"], d["b_attn"], d["W_proj"], d["b_proj"])
    torch.cuda.synchronize()
    r = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 4,
                       store_bf16=("qkv", "ym"))["y"]
    _gate(from_torch(y), r, 2.0 ** -7, 2.0 ** -8 * np.abs(r).max() + 1e-5, "plain forward")
    layer.close()


def test_block_fp32_handle_is_unsupported():
    import torch
    layer = ga.Layer(128, 4, 1, 8, "f32")
    t = torch.zeros((1, 8, 128), device="cuda")
    w = torch.zeros((128, 384), device="cuda")
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_block_forward(layer.h, t, t[0, 0], None, w, None, t[0], None, 4, t)
    assert e.value.code == ga.ERR_UNSUPPORTED
    layer.close()


def _mlp_gpu(m):
    import torch
    d = {k: to_torch(getattr(m, k), "bf16", "cuda")
         for k in ("x", "W_fc", "b_fc", "W_proj", "b_proj", "residual")}
    M, C = m.x.shape
    F = m.W_fc.shape[1]
    hbuf = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, C), dtype=torch.bfloat16, device="cuda")
    ga.gpt_mlp_forward(d["x"], d["W_fc"], d["b_fc"], d["W_proj"], d["b_proj"], hbuf, y,
                       residual=d["residual"])
    torch.cuda.synchronize()
    return from_torch(hbuf), from_torch(y)


def _mlp_check(m):
    """Activations within one bf16 ulp of the exact GELU output.  Output
    against the oracle that rounds its exact activations to bf16: where the
    GPU's fp32 pre-activation lands on the other side of a rounding boundary
    the two stored activations differ by one ulp (<= 2^-7 |h|), which moves an
    output by at most 2^-7 max|h| max|W_proj| per such activation; they are
    rare (about one in 10^4), so besides that elementwise bound at most 0.1% of
    the outputs may exceed one ulp + 1e-4, and the normwise error is <= 2^-8."""
    gh, gy = _mlp_gpu(m)
    exact = oracle.mlp_forward(m.x, m.W_fc, m.b_fc, m.W_proj, m.b_proj, want_h=True)
    _gate(gh, exact["h"], 2.0 ** -7, 1e-6, "mlp activations")
    r = oracle.mlp_forward(m.x, m.W_fc, m.b_fc, m.W_proj, m.b_proj, store_bf16=("h",))["y"]
    if m.residual is not None:
        r = r + m.residual
    flip = 2.0 ** -7 * np.abs(exact["h"]).max() * np.abs(m.W_proj).max()
    _gate(gy, r, 2.0 ** -7, flip + 1e-5, "mlp out")
    err = np.abs(gy - r)
    frac = np.mean(err > 2.0 ** -7 * np.abs(r) + 1e-4)
    assert frac <= 1e-3, f"mlp out: {frac:.2e} of the outputs beyond one ulp + 1e-4"
    rel = np.linalg.norm(gy - r) / np.linalg.norm(r)
    assert rel <= 2.0 ** -8, f"mlp out: normwise error {rel:.3e}"


@pytest.mark.parametrize("M,C,F,bias,res", [(300, 256, 1024, True, False),
                                             (257, 128, 512, False, True),
                                             (1, 64, 256, True, True),
                                             (1000, 768, 3072, True, True),
                                             # 96 x 384 c_proj tiles, ragged last row tile
                                             (7000, 768, 3072, True, True),
                                             (6600, 768, 3072, False, False),
                                             # K = F = 3000: a partial last k-tile
                                             (6600, 768, 3000, True, True)])
def test_mlp_small(M, C, F, bias, res):
    m = make_mlp_inputs(M, C, F, seed=M + F, bias=bias, with_residual=res,
                        proj_std=0.05)
    _mlp_check(m)


def test_mlp_gpt2_124m_full():
    """GPT-2 124M MLP at the layer's token count: M = 12 x 1024, C = 768,
    F = 3072, with the residual add."""
    m = make_mlp_inputs(12288, 768, 3072, seed=21, with_residual=True, proj_std=0.05)
    _mlp_check(m)


def test_mlp_gelu_negative_tail_and_zero():
    """Pre-activations spanning the GELU's regimes (large negative -> -0,
    zero -> 0, large positive -> identity) through an identity c_fc."""
    from gpt_causal_self_amd.inputs import MlpInputs, to_dtype
    C = 64
    vals = np.linspace(-12, 12, 4 * C, dtype=np.float32).reshape(4, C)
    x = to_dtype(vals, "bf16")
    eye = np.eye(C, dtype=np.float32)
    m = MlpInputs(x, eye, None, eye, None, None)
    gh, gy = _mlp_gpu(m)
    exact = oracle.mlp_forward(x, eye, None, eye, None, want_h=True)["h"]
    _gate(gh, exact, 2.0 ** -7, 1e-6, "gelu")
    assert np.array_equal(gh[x > 10], x[x > 10])     # Phi(v) rounds to 1
