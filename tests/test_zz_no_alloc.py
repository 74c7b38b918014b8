"""The allocation-free forward (gpt_attn_forward_noalloc) against the handle
forward (gpt_attn_forward), through the C ABI: the same kernels, so the same
outputs bit for bit, on consecutive calls that share the static scratch --
the GPT-2 124M workload first, then smaller inputs (a ragged multi-tile
shape, head size 32, a split-K short sequence, one position) -- and the
stated bf16 tolerance against the oracle on one of them.  Sizes beyond the
scratch are rejected before any device work."""
from __future__ import annotations

import numpy as np
import pytest

from gpt_causal_self_amd import gpt_attn as ga
from gpt_causal_self_amd.inputs import from_torch, make_inputs, workload_inputs
from layer_helpers import assert_close, device_inputs, oracle_forward

pytestmark = pytest.mark.gpu


def _both(inp):
    import torch
    B, T, C = inp.x.shape
    H = inp.n_head
    t = device_inputs(inp)
    layer = ga.Layer(C, H, B, T, "bf16")
    ref = layer.forward(t["x"], t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"])
    y = torch.full_like(t["x"], float("nan"))
    ga.gpt_attn_forward_noalloc(t["x"], t["W_attn"], t["b_attn"], t["W_proj"], t["b_proj"],
                                H, y)
    torch.cuda.synchronize()
    layer.close()
    return from_torch(y), from_torch(ref)


def test_noalloc_matches_the_handle_forward_on_consecutive_calls():
    cases = [workload_inputs(2),                                           # 75.5 MB of scratch
             make_inputs(2, 300, 768, 12, dtype="bf16", seed=61),        # smaller, ragged
             make_inputs(3, 200, 256, 8, dtype="bf16", seed=62),         # hs 32
             make_inputs(4, 128, 1600, 25, bias=False, dtype="bf16", seed=63),  # split-K
             make_inputs(5, 1, 128, 2, dtype="bf16", seed=64)]           # one position
    for i, inp in enumerate(cases):
        g, r = _both(inp)
        assert np.array_equal(g, r), f"case {i}: differs from gpt_attn_forward"
        if i == 1:
            assert_close(g, oracle_forward(inp)["y"], "bf16", "noalloc forward")


def test_noalloc_rejects_what_does_not_fit_and_bad_arguments():
    import torch
    C, H = 768, 12
    x = torch.zeros((1, 16, C), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((C, 3 * C), dtype=torch.bfloat16, device="cuda")
    Wp = torch.zeros((C, C), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    need = 4 * 16 * 1024 * C * 2            # B = 16, T = 1024: 100.7 MB > 80 MiB
    assert need > ga.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_forward_noalloc(x, W, None, Wp, None, H, y, B=16, T=1024, C=C)
    assert e.value.code == ga.ERR_SHAPE
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_forward_noalloc(x, W, None, Wp, None, 5, y)      # C % n_head != 0
    assert e.value.code == ga.ERR_SHAPE
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_forward_noalloc(x, W, None, Wp, None, 6, y)      # hs = 128
    assert e.value.code == ga.ERR_UNSUPPORTED
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_forward_noalloc(None, W, None, Wp, None, H, y, B=1, T=16, C=C)
    assert e.value.code == ga.ERR_INVALID_ARG
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_forward_noalloc(x.data_ptr() + 2, W, None, Wp, None, H, y, B=1, T=16, C=C)
    assert e.value.code == ga.ERR_ALIGN
    ga.gpt_attn_forward_noalloc(x, W, None, Wp, None, H, y, B=0, T=16, C=C)   # no-op
    torch.cuda.synchronize()
