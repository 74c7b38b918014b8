"""GPU parity of the training-time dropout (gpt_attn_set_dropout) against the
fp64 oracle replaying the same Philox4x32-10 masks.

The keep decisions are integer comparisons of generator words with the same
threshold on both sides, so the masks agree exactly; what remains is the
rounding of the bf16 path, judged with the oracle that rounds q/k/v and the
merged heads like the GPU (one ulp of the output plus 2^-8 of the row's
largest output).  Dropped c_proj outputs are exactly zero on both sides,
which checks the output mask bit for bit (a kept output can also be zero on
the GPU, where its fp32 accumulator cancels the bias exactly: those few sit
inside the rounding gate)."""
from __future__ import annotations

import numpy as np
import pytest

import grad_gate
import oracle
from gpt_causal_self_amd import gpt_attn as ga
from gpt_causal_self_amd.inputs import from_torch, make_inputs, make_ln_params, to_torch

pytestmark = pytest.mark.gpu


def _inputs(B, T, C, H, seed, bias=True):
    return make_inputs(B, T, C, H, bias=bias, dtype="bf16", seed=seed, proj_std=0.2,
                       b_proj_std=0.2 if bias else 0.0)


def _fwd(inp, p, seed, layer=None, save=False):
    import torch
    B, T, C = inp.x.shape
    own = layer is None
    if own:
        layer = ga.Layer(C, inp.n_head, B, T, "bf16")
    d = {k: to_torch(getattr(inp, k), "bf16", "cuda")
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    ga.gpt_attn_set_dropout(layer.h, p, seed)
    y = layer.forward(d["x"], d["W_attn"], d["b_attn"], d["W_proj"], d["b_proj"],
                      save_for_backward=save)
    torch.cuda.synchronize()
    out = from_torch(y)
    if own:
        layer.close()
    return out


def _check(g, r, what):
    scale = np.abs(r).max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    bound = 2.0 ** -7 * np.abs(r) + 2.0 ** -8 * scale + 1e-5
    if not np.all(err <= bound):
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {(err > bound).sum()} out of the gate; worst at {idx}: "
                             f"got {g[idx]!r} want {r[idx]!r} (bound {bound[idx]:.3e})")
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    assert rel < 4e-3, f"{what}: normwise error {rel:.3e}"
    # every output the oracle drops is exactly zero on the GPU
    dropped = r == 0.0
    assert np.all(g[dropped] == 0.0), f"{what}: {(g[dropped] != 0.0).sum()} dropped outputs kept"
    # a kept output is exactly zero on the GPU only where its fp32 accumulator
    # cancels the bias exactly; the gate above admits that only within rounding
    # of zero, and it is rare (about one output in 10^7 at the 124M shape)
    extra = int(((g == 0.0) & ~dropped).sum())
    assert extra <= max(2, g.size // 1_000_000), f"{what}: {extra} kept outputs are zero"


@pytest.mark.parametrize("B,T,C,H,p,seed", [(2, 70, 256, 4, 0.1, 1), (3, 129, 128, 4, 0.5, 2),
                                            (1, 64, 256, 8, 0.9, 3),
                                            # 7000 rows at C = 768: the c_proj of 96 x 384
                                            # tiles with a ragged last row tile
                                            (7, 1000, 768, 12, 0.1, 4)])
def test_dropout_forward_small(B, T, C, H, p, seed):
    inp = _inputs(B, T, C, H, seed=T + C)
    g = _fwd(inp, p, seed)
    r = oracle.forward_dropout(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                               np.float32(p), seed, store_bf16=("qkv", "ym"))["y"]
    _check(g, r, "dropout forward")


def test_dropout_forward_gpt2_124m_full():
    """GPT-2 124M shape, p = 0.1 (the dropout of one page's training
    configuration), a 64-bit seed."""
    inp = _inputs(12, 1024, 768, 12, seed=8)
    seed = 0x1234_5678_9ABC_DEF0
    g = _fwd(inp, 0.1, seed)
    r = oracle.forward_dropout(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 12,
                               np.float32(0.1), seed, store_bf16=("qkv", "ym"))["y"]
    _check(g, r, "dropout forward 124M")


def test_zero_rate_is_the_plain_forward_bitwise():
    import torch
    inp = _inputs(2, 96, 256, 4, seed=4)
    layer = ga.Layer(256, 4, 2, 96, "bf16")
    d = {k: to_torch(getattr(inp, k), "bf16", "cuda")
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    plain = from_torch(layer.forward(d["x"], d["W_attn"], d["b_attn"], d["W_proj"], d["b_proj"]))
    torch.cuda.synchronize()
    assert np.array_equal(_fwd(inp, 0.0, 5, layer=layer), plain)
    layer.close()


def test_seed_determines_the_masks():
    inp = _inputs(2, 64, 128, 4, seed=6)
    a, b, c = _fwd(inp, 0.3, 10), _fwd(inp, 0.3, 10), _fwd(inp, 0.3, 11)
    assert np.array_equal(a, b)
    assert np.mean(a != c) > 0.2


def test_block_forward_with_dropout():
    import torch
    B, T, C, H = 2, 80, 256, 4
    inp = _inputs(B, T, C, H, seed=12)
    ln_w, ln_b = make_ln_params(C, seed=13)
    layer = ga.Layer(C, H, B, T, "bf16")
    ga.gpt_attn_set_dropout(layer.h, 0.2, 21)
    d = {k: to_torch(getattr(inp, k), "bf16", "cuda")
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    out = torch.empty_like(d["x"])
    ga.gpt_attn_block_forward(layer.h, d["x"], to_torch(ln_w, "bf16", "cuda"),
                              to_torch(ln_b, "bf16", "cuda"), d["W_attn"], d["b_attn"],
                              d["W_proj"], d["b_proj"], H, out)
    torch.cuda.synchronize()
    layer.close()
    ln = oracle.block_attn_forward(inp.x, ln_w, ln_b, inp.W_attn, inp.b_attn, inp.W_proj,
                                   inp.b_proj, H, want_ln=True, store_bf16=("ln",))["ln"]
    y = oracle.forward_dropout(ln, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                               np.float32(0.2), 21, store_bf16=("qkv", "ym"))["y"]
    r = inp.x + y
    g = from_torch(out)
    scale = np.abs(y).max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    assert np.all(err <= 2.0 ** -7 * np.abs(r) + 2.0 ** -8 * scale + 1e-5), err.max()


def test_dropout_errors():
    import torch
    layer = ga.Layer(128, 4, 1, 16, "bf16")
    for bad in (1.0, -0.1, float("nan")):
        with pytest.raises(ga.GptAttnError) as e:
            ga.gpt_attn_set_dropout(layer.h, bad, 0)
        assert e.value.code == ga.ERR_INVALID_ARG
    layer.close()
    f32 = ga.Layer(128, 4, 1, 16, "f32")
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_set_dropout(f32.h, 0.1, 0)
    assert e.value.code == ga.ERR_UNSUPPORTED
    ga.gpt_attn_set_dropout(f32.h, 0.0, 0)        # switching off is always allowed
    f32.close()


@pytest.mark.parametrize("B,T,C,H,p,seed", [(2, 70, 256, 4, 0.1, 31), (1, 129, 128, 4, 0.5, 32),
                                            (2, 1024, 768, 12, 0.1, 33)])
def test_dropout_backward(B, T, C, H, p, seed):
    """Gradients of a dropout forward against the oracle's gradient through
    the same masks: the stated tolerance elementwise against the oracle with
    the bf16 path's roundings, normwise 1e-2 against the exact one."""
    import torch
    inp = make_inputs(B, T, C, H, dtype="bf16", seed=T + seed, with_dY=True)
    layer = ga.Layer(C, H, B, T, "bf16")
    d = {k: to_torch(getattr(inp, k), "bf16", "cuda")
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj", "dY")}
    ga.gpt_attn_set_dropout(layer.h, p, seed)
    layer.forward(d["x"], d["W_attn"], d["b_attn"], d["W_proj"], d["b_proj"],
                  save_for_backward=True)
    g = {k: from_torch(v) for k, v in
         layer.backward(d["x"], d["W_attn"], d["W_proj"], d["dY"]).items()}
    torch.cuda.synchronize()
    layer.close()
    grad_gate.check_all(g, inp, p=float(np.float32(p)), seed=seed)


@pytest.mark.parametrize("C,H", [(256, 4), (128, 4)])
def test_dropout_backward_below_the_handle_maxima(C, H):
    """Dropout gradients on a handle created for larger B and T than the call
    (the stored keep bits are laid out for the call's T inside a buffer sized
    for the maxima), after a first training step at another shape on the same
    handle, against the oracle's exact gradient through the same masks."""
    import torch
    p = 0.2
    layer = ga.Layer(C, H, 3, 400, "bf16")
    for (B, T, seed) in ((3, 400, 51), (2, 257, 52)):
        inp = make_inputs(B, T, C, H, dtype="bf16", seed=T + seed, with_dY=True)
        d = {k: to_torch(getattr(inp, k), "bf16", "cuda")
             for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj", "dY")}
        ga.gpt_attn_set_dropout(layer.h, p, seed)
        layer.forward(d["x"], d["W_attn"], d["b_attn"], d["W_proj"], d["b_proj"],
                      save_for_backward=True)
        g = {k: from_torch(v) for k, v in
             layer.backward(d["x"], d["W_attn"], d["W_proj"], d["dY"]).items()}
        torch.cuda.synchronize()
        grad_gate.check_all(g, inp, p=float(np.float32(p)), seed=seed)
    layer.close()
