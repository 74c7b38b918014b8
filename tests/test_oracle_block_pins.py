"""Pins of the oracle's LayerNorm, Pre-LN attention half-block and MLP.

Tied to: torch fp64 library routines (F.layer_norm, F.gelu with the exact
erf form, the layer composed from F.linear + causal SDPA); closed forms (a
constant row normalises to the bias; gelu(u) - gelu(-u) = u; gelu(1) equals
the standard normal CDF at 1; identity weights turn the MLP into gelu); and
invariants (zero c_proj weights make the block the identity on x)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from gpt_causal_self_amd.inputs import make_inputs


def _t(a):
    import torch
    return None if a is None else torch.from_numpy(np.asarray(a, np.float64))


@pytest.mark.parametrize("bias", [True, False])
def test_layernorm_matches_torch(bias):
    import torch.nn.functional as F
    rng = np.random.default_rng(0)
    x = rng.standard_normal((37, 96)) * 3 + 1.5
    w = rng.standard_normal(96)
    b = rng.standard_normal(96) if bias else None
    got = oracle.layernorm(x, w, b)
    ref = F.layer_norm(_t(x), (96,), _t(w), _t(b), 1e-5).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_layernorm_closed_forms():
    rng = np.random.default_rng(1)
    C = 64
    x = rng.standard_normal((5, C))
    x[0] = 2.5                                   # constant row -> bias
    w = np.ones(C)
    b = np.linspace(-1, 1, C)
    out = oracle.layernorm(x, w, b)
    np.testing.assert_allclose(out[0], b, rtol=0, atol=1e-15)
    z = oracle.layernorm(x[1:], w, None)
    np.testing.assert_allclose(z.mean(-1), 0.0, atol=1e-14)
    v = x[1:].var(-1)
    np.testing.assert_allclose((z ** 2).mean(-1), v / (v + 1e-5), rtol=1e-12)


def _mlp_identity(u):
    C = u.shape[-1]
    eye = np.eye(C)
    return oracle.mlp_forward(u, eye, None, eye, None)["y"]


def test_gelu_closed_forms():
    u = np.linspace(-6, 6, 97).reshape(1, 97)
    g = _mlp_identity(u)
    gm = _mlp_identity(-u)
    np.testing.assert_allclose(g - gm, u, rtol=0, atol=1e-14)
    one = _mlp_identity(np.array([[1.0, 0.0, -1.0]]))
    phi1 = 0.5 * (1 + math.erf(1 / math.sqrt(2)))         # standard normal CDF at 1
    assert abs(one[0, 0] - phi1) < 1e-15 and abs(phi1 - 0.8413447460685429) < 1e-15
    assert one[0, 1] == 0.0


def test_gelu_matches_torch_exact_form():
    import torch.nn.functional as F
    u = np.random.default_rng(2).standard_normal((3, 50)) * 2
    np.testing.assert_allclose(_mlp_identity(u), F.gelu(_t(u), approximate="none").numpy(),
                               rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("bias", [True, False])
def test_mlp_matches_torch(bias):
    import torch.nn.functional as F
    rng = np.random.default_rng(3)
    M, C, Fh = 29, 48, 192
    x = rng.standard_normal((M, C))
    Wf, Wp = rng.standard_normal((C, Fh)) * 0.2, rng.standard_normal((Fh, C)) * 0.1
    bf = rng.standard_normal(Fh) * 0.1 if bias else None
    bp = rng.standard_normal(C) * 0.1 if bias else None
    got = oracle.mlp_forward(x, Wf, bf, Wp, bp, want_h=True)
    h = F.gelu(F.linear(_t(x), _t(Wf).T, _t(bf)))
    ref = F.linear(h, _t(Wp).T, _t(bp)).numpy()
    np.testing.assert_allclose(got["y"], ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["h"], h.numpy(), rtol=1e-12, atol=1e-14)


def test_block_matches_torch_composition():
    import torch
    import torch.nn.functional as F
    B, T, C, H = 2, 21, 64, 4
    inp = make_inputs(B, T, C, H, dtype="f32", seed=5, w_std=0.1, proj_std=0.1)
    rng = np.random.default_rng(6)
    ln_w, ln_b = 1 + 0.1 * rng.standard_normal(C), 0.1 * rng.standard_normal(C)
    got = oracle.block_attn_forward(inp.x, ln_w, ln_b, inp.W_attn, inp.b_attn, inp.W_proj,
                                    inp.b_proj, H)["out"]
    x = _t(inp.x)
    ln = F.layer_norm(x, (C,), _t(ln_w), _t(ln_b), 1e-5)
    qkv = F.linear(ln, _t(inp.W_attn).T, _t(inp.b_attn))
    q, k, v = [a.view(B, T, H, C // H).transpose(1, 2) for a in qkv.split(C, 2)]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    y = F.linear(o.transpose(1, 2).reshape(B, T, C), _t(inp.W_proj).T, _t(inp.b_proj))
    np.testing.assert_allclose(got, (x + y).numpy(), rtol=1e-11, atol=1e-12)


def test_block_with_zero_projection_is_identity():
    B, T, C, H = 2, 9, 32, 2
    inp = make_inputs(B, T, C, H, dtype="f32", seed=7, w_std=0.3)
    out = oracle.block_attn_forward(inp.x, np.ones(C), None, inp.W_attn, inp.b_attn,
                                    np.zeros((C, C)), np.zeros(C), H)["out"]
    assert np.array_equal(out, inp.x.astype(np.float64))


def test_block_store_ln_rounds_the_layer_input():
    from test_oracle_pins import _bits_rne_bf16
    B, T, C, H = 1, 7, 32, 2
    inp = make_inputs(B, T, C, H, dtype="f32", seed=8, w_std=0.3)
    a = oracle.block_attn_forward(inp.x, np.ones(C), None, inp.W_attn, inp.b_attn,
                                  inp.W_proj, inp.b_proj, H, want_ln=True)
    b = oracle.block_attn_forward(inp.x, np.ones(C), None, inp.W_attn, inp.b_attn,
                                  inp.W_proj, inp.b_proj, H, want_ln=True, store_bf16=("ln",))
    assert np.array_equal(b["ln"], _bits_rne_bf16(a["ln"]))
    y = oracle.forward(b["ln"], inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H)["y"]
    np.testing.assert_allclose(b["out"], inp.x + y, rtol=1e-14, atol=1e-15)
