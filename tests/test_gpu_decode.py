"""GPU parity of the one-token decode with a key/value cache (through the C
ABI, include/gpt_decode.h).

The layer is causal, so decoding position t against the cached keys and
values of positions < t must give row t of the full forward.  Reference: the
fp64 oracle's full forward over the same prefix, with q/k/v and the merged
heads rounded to bf16 as the GPU stores them; gate: one bf16 ulp of the
output plus 2^-8 of the row's largest output (the attention stage's own
rounding), and a normwise gate.  The caches are checked against the
oracle's exact keys and values within one bf16 ulp."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpt_causal_self_amd import gpt_attn as ga
from gpt_causal_self_amd.inputs import from_torch, make_inputs, to_torch

pytestmark = pytest.mark.gpu


def _inputs(B, T, C, H, seed, bias=True):
    return make_inputs(B, T, C, H, bias=bias, dtype="bf16", seed=seed, proj_std=0.2,
                       b_proj_std=0.2 if bias else 0.0)


def _dev(inp):
    return {k: to_torch(getattr(inp, k), "bf16", "cuda")
            for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}


def _decode_range(layer, d, H, kc, vc, t0, t1):
    """Decode positions t0..t1-1 of x one at a time; returns y [B, t1-t0, C]."""
    import torch
    B, _, C = d["x"].shape
    ys = []
    for t in range(t0, t1):
        xt = d["x"][:, t].contiguous()
        y = torch.empty((B, C), dtype=torch.bfloat16, device="cuda")
        ga.gpt_attn_decode(layer.h, xt, d["W_attn"], d["b_attn"], d["W_proj"], d["b_proj"], H,
                           kc, vc, y, t)
        ys.append(y)
    torch.cuda.synchronize()
    return np.stack([from_torch(y) for y in ys], axis=1)


def _check_rows(g, inp, t0, t1):
    r = oracle.forward(inp.x[:, :t1], inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                       inp.n_head, store_bf16=("qkv", "ym"))["y"][:, t0:t1]
    scale = np.abs(r).max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    bound = 2.0 ** -7 * np.abs(r) + 2.0 ** -8 * scale + 1e-5
    if not np.all(err <= bound):
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"decode rows: {(err > bound).sum()} out of the gate; worst at "
                             f"{idx}: got {g[idx]!r} want {r[idx]!r} (bound {bound[idx]:.3e})")
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    assert rel < 4e-3, f"decode rows: normwise error {rel:.3e}"


def _check_cache(kc, vc, inp, T):
    B, _, C = inp.x.shape
    H = inp.n_head
    hs = C // H
    qkv = oracle.forward(inp.x[:, :T], inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                         want=("qkv",))["qkv"]
    for s, cache in ((1, kc), (2, vc)):
        r = qkv[:, :, s * C:(s + 1) * C].reshape(B, T, H, hs).transpose(0, 2, 1, 3)
        g = from_torch(cache)[:, :, :T]
        err = np.abs(g - r)
        assert np.all(err <= 2.0 ** -7 * np.abs(r) + 1e-6), ("kv cache", s, err.max())


@pytest.mark.parametrize("B,T,C,H", [(2, 70, 128, 4), (3, 40, 256, 4), (1, 300, 256, 4)])
def test_decode_from_empty_cache_matches_full_forward(B, T, C, H):
    import torch
    inp = _inputs(B, T, C, H, seed=T + C)
    d = _dev(inp)
    hs = C // H
    layer = ga.Layer(C, H, B, T, "bf16")
    kc = torch.zeros((B, H, T, hs), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    g = _decode_range(layer, d, H, kc, vc, 0, T)
    layer.close()
    _check_rows(g, inp, 0, T)
    _check_cache(kc, vc, inp, T)


def test_prefill_then_decode():
    """Full forward over the first 50 positions, export of its keys and
    values, then decode of positions 50..99 into a longer cache."""
    import torch
    B, T0, T, C, H = 3, 50, 100, 256, 4
    inp = _inputs(B, T, C, H, seed=5, bias=False)
    d = _dev(inp)
    layer = ga.Layer(C, H, B, T, "bf16")
    y0 = torch.empty((B, T0, C), dtype=torch.bfloat16, device="cuda")
    ga.gpt_attn_forward(layer.h, d["x"][:, :T0].contiguous(), d["W_attn"], d["b_attn"],
                        d["W_proj"], d["b_proj"], H, y0, B=B, T=T0)
    kc = torch.full((B, H, 128, C // H), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    ga.gpt_attn_export_kv(layer.h, kc, vc)
    g = _decode_range(layer, d, H, kc, vc, T0, T)
    layer.close()
    _check_rows(g, inp, T0, T)
    _check_cache(kc, vc, inp, T)
    assert torch.isnan(kc[:, :, T:].float()).all()        # untouched beyond T


def test_decode_gpt2_124m_shape_across_chunk_boundaries():
    """GPT-2 124M attention shape (12 sequences, C=768, 12 heads): prefill
    250 positions, then decode 250..265 and 508..520 after a second
    prefill."""
    import torch
    B, T, C, H = 12, 521, 768, 12
    inp = _inputs(B, T, C, H, seed=77)
    d = _dev(inp)
    layer = ga.Layer(C, H, B, T, "bf16")
    kc = torch.zeros((B, H, 1024, C // H), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for t0, t1 in ((250, 266), (508, 521)):
        y0 = torch.empty((B, t0, C), dtype=torch.bfloat16, device="cuda")
        ga.gpt_attn_forward(layer.h, d["x"][:, :t0].contiguous(), d["W_attn"], d["b_attn"],
                            d["W_proj"], d["b_proj"], H, y0, B=B, T=t0)
        ga.gpt_attn_export_kv(layer.h, kc, vc)
        g = _decode_range(layer, d, H, kc, vc, t0, t1)
        _check_rows(g, inp, t0, t1)
    layer.close()


@pytest.mark.parametrize("C,H", [(128, 4), (256, 4)])
def test_decode_across_attention_blocks(C, H):
    """Caches longer than one attention block (1024 keys): prefill 1021
    positions, then decode 1021..1027, so that the keys of one query span one
    and then two blocks whose partial results are merged (head sizes 32, 64)."""
    import torch
    B, T, T0 = 2, 1028, 1021
    inp = _inputs(B, T, C, H, seed=31)
    d = _dev(inp)
    layer = ga.Layer(C, H, B, T, "bf16")
    kc = torch.zeros((B, H, 1100, C // H), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    y0 = torch.empty((B, T0, C), dtype=torch.bfloat16, device="cuda")
    ga.gpt_attn_forward(layer.h, d["x"][:, :T0].contiguous(), d["W_attn"], d["b_attn"],
                        d["W_proj"], d["b_proj"], H, y0, B=B, T=T0)
    ga.gpt_attn_export_kv(layer.h, kc, vc)
    g = _decode_range(layer, d, H, kc, vc, T0, T)
    layer.close()
    _check_rows(g, inp, T0, T)


def test_decode_is_deterministic():
    import torch
    B, T, C, H = 2, 33, 128, 4
    inp = _inputs(B, T, C, H, seed=9)
    d = _dev(inp)
    outs = []
    for _ in range(2):
        layer = ga.Layer(C, H, B, T, "bf16")
        kc = torch.zeros((B, H, T, C // H), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        outs.append(_decode_range(layer, d, H, kc, vc, 0, T))
        layer.close()
    assert np.array_equal(outs[0], outs[1])


def test_decode_and_export_errors():
    import torch
    C, H = 128, 4
    layer = ga.Layer(C, H, 2, 16, "bf16")
    kc = torch.zeros((2, H, 16, C // H), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((2, C), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((C, 3 * C), dtype=torch.bfloat16, device="cuda")
    Wp = torch.zeros((C, C), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(ga.GptAttnError) as e:           # no forward yet
        ga.gpt_attn_export_kv(layer.h, kc, kc)
    assert e.value.code == ga.ERR_STATE
    with pytest.raises(ga.GptAttnError) as e:           # pos beyond the cache
        ga.gpt_attn_decode(layer.h, x, W, None, Wp, None, H, kc, kc, y, 16)
    assert e.value.code == ga.ERR_INVALID_ARG
    with pytest.raises(ga.GptAttnError) as e:           # B above the handle's max
        ga.gpt_attn_decode(layer.h, torch.zeros((3, C), dtype=torch.bfloat16, device="cuda"),
                           W, None, Wp, None, H, kc, kc, torch.empty((3, C), dtype=torch.bfloat16,
                                                                      device="cuda"), 0)
    assert e.value.code == ga.ERR_SHAPE
    xs = torch.zeros((2, 16, C), dtype=torch.bfloat16, device="cuda")
    ga.gpt_attn_forward(layer.h, xs, W, None, Wp, None, H, torch.empty_like(xs))
    with pytest.raises(ga.GptAttnError) as e:           # cache shorter than T
        ga.gpt_attn_export_kv(layer.h, kc, kc, cache_T=8)
    assert e.value.code == ga.ERR_SHAPE
    ga.gpt_attn_decode(layer.h, x, W, None, Wp, None, H, kc, kc, y, 3)
    with pytest.raises(ga.GptAttnError) as e:           # decode dropped the forward's q/k/v
        ga.gpt_attn_export_kv(layer.h, kc, kc)
    assert e.value.code == ga.ERR_STATE
    torch.cuda.synchronize()
    layer.close()
    f32 = ga.Layer(C, H, 2, 16, "f32")
    with pytest.raises(ga.GptAttnError) as e:
        ga.gpt_attn_decode(f32.h, x, W, None, Wp, None, H, kc, kc, y, 0)
    assert e.value.code == ga.ERR_UNSUPPORTED
    f32.close()
