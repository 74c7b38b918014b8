"""Every output buffer is written exactly where its shape says, nothing
around it: each output lives inside a larger buffer whose guard bands hold a
sentinel, and the sentinels must survive the call (gradients of the training
step, the block and MLP outputs, the decode output and the key/value caches,
whose rows other than the decoded position must stay as they were)."""
from __future__ import annotations

import numpy as np
import pytest

from gpt_causal_self_amd import gpt_attn as ga
from gpt_causal_self_amd.inputs import make_inputs, make_ln_params, make_mlp_inputs, to_torch
from layer_helpers import device_inputs

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 7.0


def _guarded(shape, dtype):
    """(view of the requested shape, whole buffer) with sentinels around."""
    import torch
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=dtype, device="cuda")
    return buf[GUARD:GUARD + n].view(*shape), buf


def _guards_intact(buf, n, what):
    import torch
    assert torch.all(buf[:GUARD] == SENTINEL), f"{what}: guard band before the output written"
    assert torch.all(buf[GUARD + n:] == SENTINEL), f"{what}: guard band after the output written"


@pytest.mark.parametrize("B,T,C,H,dtype,drop", [(3, 77, 256, 4, "bf16", 0.0),
                                                (2, 130, 768, 12, "bf16", 0.1),
                                                (2, 45, 128, 2, "f32", 0.0)])
def test_backward_outputs_stay_in_bounds(B, T, C, H, dtype, drop):
    import torch
    inp = make_inputs(B, T, C, H, dtype=dtype, seed=B + T, with_dY=True)
    t = device_inputs(inp)
    td = t["x"].dtype
    layer = ga.Layer(C, H, B + 1, T + 20, dtype)
    if drop:
        ga.gpt_attn_set_dropout(layer.h, drop, 17)
    layer.forward(t["x"], t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"],
                  save_for_backward=True)
    shapes = {"dx": (B, T, C), "dW_attn": (C, 3 * C), "db_attn": (3 * C,),
              "dW_proj": (C, C), "db_proj": (C,)}
    out = {k: _guarded(s, td) for k, s in shapes.items()}
    ga.gpt_attn_backward(layer.h, t["x"], t["W_attn"], t["W_proj"], t["dY"],
                         out["dx"][0], out["dW_attn"][0], out["db_attn"][0],
                         out["dW_proj"][0], out["db_proj"][0])
    torch.cuda.synchronize()
    # the same step into plain tensors gives the same gradients (bitwise)
    layer.forward(t["x"], t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"],
                  save_for_backward=True)
    ref = layer.backward(t["x"], t["W_attn"], t["W_proj"], t["dY"])
    torch.cuda.synchronize()
    layer.close()
    for k, (view, buf) in out.items():
        _guards_intact(buf, view.numel(), k)
        assert torch.equal(view, ref[k]), k


def test_block_and_mlp_outputs_stay_in_bounds():
    import torch
    B, T, C, H = 2, 90, 256, 4
    inp = make_inputs(B, T, C, H, dtype="bf16", seed=3)
    t = device_inputs(inp)
    ln_w, ln_b = make_ln_params(C, seed=4)
    layer = ga.Layer(C, H, B, T, "bf16")
    out, buf = _guarded((B, T, C), torch.bfloat16)
    ga.gpt_attn_block_forward(layer.h, t["x"], to_torch(ln_w, "bf16", "cuda"),
                              to_torch(ln_b, "bf16", "cuda"), t["W_attn"], t["b_attn"],
                              t["W_proj"], t["b_proj"], H, out)
    torch.cuda.synchronize()
    layer.close()
    _guards_intact(buf, out.numel(), "block output")
    assert torch.isfinite(out.float()).all()
    M, F = 150, 1024
    m = make_mlp_inputs(M, C, F, seed=5, with_residual=True)
    d = {k: to_torch(getattr(m, k), "bf16", "cuda")
         for k in ("x", "W_fc", "b_fc", "W_proj", "b_proj", "residual")}
    hb, hbuf = _guarded((M, F), torch.bfloat16)
    y, ybuf = _guarded((M, C), torch.bfloat16)
    ga.gpt_mlp_forward(d["x"], d["W_fc"], d["b_fc"], d["W_proj"], d["b_proj"], hb, y,
                       residual=d["residual"])
    torch.cuda.synchronize()
    _guards_intact(hbuf, hb.numel(), "MLP activations")
    _guards_intact(ybuf, y.numel(), "MLP output")


@pytest.mark.parametrize("cache_T,pos", [(64, 40), (1100, 1030)])
def test_decode_outputs_and_caches_stay_in_bounds(cache_T, pos):
    """One decode step at pos writes y and cache position pos of every
    (b, h) row, and nothing else."""
    import torch
    B, C, H = 3, 256, 4
    hs = C // H
    inp = make_inputs(B, pos + 1, C, H, dtype="bf16", seed=pos)
    t = device_inputs(inp)
    layer = ga.Layer(C, H, B, pos + 1, "bf16")
    g = torch.Generator(device="cuda").manual_seed(1)
    kc, kbuf = _guarded((B, H, cache_T, hs), torch.bfloat16)
    vc, vbuf = _guarded((B, H, cache_T, hs), torch.bfloat16)
    kc.copy_(torch.randn(kc.shape, generator=g, device="cuda").to(torch.bfloat16))
    vc.copy_(torch.randn(vc.shape, generator=g, device="cuda").to(torch.bfloat16))
    k0, v0 = kc.clone(), vc.clone()
    y, ybuf = _guarded((B, C), torch.bfloat16)
    ga.gpt_attn_decode(layer.h, t["x"][:, pos].contiguous(), t["W_attn"], t["b_attn"],
                       t["W_proj"], t["b_proj"], H, kc, vc, y, pos)
    torch.cuda.synchronize()
    layer.close()
    _guards_intact(ybuf, y.numel(), "decode output")
    _guards_intact(kbuf, kc.numel(), "key cache")
    _guards_intact(vbuf, vc.numel(), "value cache")
    keep = torch.ones(cache_T, dtype=torch.bool, device="cuda")
    keep[pos] = False
    assert torch.equal(kc[:, :, keep], k0[:, :, keep]), "key cache rows other than pos changed"
    assert torch.equal(vc[:, :, keep], v0[:, :, keep]), "value cache rows other than pos changed"
    assert not torch.equal(kc[:, :, pos], k0[:, :, pos])
    assert torch.isfinite(y.float()).all()
