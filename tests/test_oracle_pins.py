"""Pins of the CPU oracle against what the pages and mathematics fix.

The oracle (``oracle/``) is the definition of causal self-attention written
out in fp64.  These CPU tests tie it to things other than itself:
  * brute force: pure-Python loops (``oracle/brute.py``) on tiny shapes;
  * library special case: torch CPU fp64 ``F.linear`` + causal
    ``scaled_dot_product_attention``, and the pages' manual masked-softmax
    form, plus torch autograd for the backward;
  * closed forms and invariants: rows of P sum to 1, zero weight on future
    positions, causality (bitwise), T = 1 reduces to c_proj(v), constant
    sequences, the uniform-attention prefix mean, prefix permutation, head
    permutation and batch independence;
  * finite differences for the backward;
  * the weight sizes printed on page "nanoGPT architecture explained step by
    step", parameter-count table (``tests/golden/param_counts.txt``).
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
import oracle.brute as brute
from gpt_causal_self_amd.inputs import WORKLOADS, make_inputs, workload_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fwd(inp, want=("y",), lib=None):
    return oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                          inp.n_head, want=want, lib=lib)


def tiny(B=2, T=7, C=8, H=2, bias=True, seed=0, **kw):
    kw.setdefault("w_std", 0.5)
    kw.setdefault("proj_std", 0.5)
    kw.setdefault("b_attn_std", 0.3)
    kw.setdefault("b_proj_std", 0.3)
    return make_inputs(B, T, C, H, bias=bias, dtype="f32", seed=seed, **kw)


# ---------------------------------------------------------------- I1 shapes
def test_param_counts_match_pages():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "param_counts.txt"))
            if l.strip() and not l.startswith("#")]
    w = workload_inputs(2, B=1, T=1)
    got = {"c_attn": w.W_attn.shape, "c_proj": w.W_proj.shape}
    for name, r, c, approx in rows:
        assert got[name] == (int(r), int(c))
        assert round(int(r) * int(c) / 1e6, 2) == float(approx)


def test_output_shapes():
    inp = tiny(B=3, T=5, C=12, H=3)
    o = fwd(inp, want=("y", "qkv", "ym", "P", "lse"))
    assert o["y"].shape == (3, 5, 12)
    assert o["qkv"].shape == (3, 5, 36)
    assert o["ym"].shape == (3, 5, 12)
    assert o["P"].shape == (3, 3, 5, 5)
    assert o["lse"].shape == (3, 3, 5)


# ------------------------------------------------------------ brute force
@pytest.mark.parametrize("B,T,C,H,bias", [
    (1, 1, 4, 1, True), (2, 5, 8, 2, True), (2, 9, 16, 4, False),
    (1, 9, 16, 1, True), (2, 3, 12, 3, True)])
def test_brute_force(B, T, C, H, bias):
    inp = tiny(B, T, C, H, bias=bias, seed=B * 100 + T)
    o = fwd(inp, want=("y", "P", "lse"))
    yb, Pb = brute.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj,
                           inp.b_proj, H)
    np.testing.assert_allclose(o["y"], np.array(yb), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o["P"], np.array(Pb), rtol=1e-12, atol=1e-15)
    # log-sum-exp of the scaled, visible scores, straight from the formula
    q = o_qkv = fwd(inp, want=("qkv",))["qkv"]
    hs = C // H
    for b in range(B):
        for h in range(H):
            for i in range(T):
                s = [sum(q[b, i, h * hs + d] * o_qkv[b, j, C + h * hs + d]
                         for d in range(hs)) / math.sqrt(hs) for j in range(i + 1)]
                lse = math.log(sum(math.exp(v) for v in s))
                assert abs(o["lse"][b, h, i] - lse) <= 1e-12 * max(1, abs(lse))


# ------------------------------------------------------ library special case
def _torch_layer(inp, manual=False):
    import torch
    import torch.nn.functional as F
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float64))  # noqa
    x, Wa, ba, Wp, bp = map(t, (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj))
    B, T, C = x.shape
    H = inp.n_head
    hs = C // H
    qkv = F.linear(x, Wa.T, ba)
    q, k, v = qkv.split(C, dim=2)
    q = q.view(B, T, H, hs).transpose(1, 2)
    k = k.view(B, T, H, hs).transpose(1, 2)
    v = v.view(B, T, H, hs).transpose(1, 2)
    if manual:
        att = (q @ k.transpose(-2, -1)) * (1.0 / math.sqrt(hs))
        mask = torch.tril(torch.ones(T, T, dtype=torch.float64)).view(1, 1, T, T)
        att = att.masked_fill(mask == 0, float("-inf"))
        att = F.softmax(att, dim=-1)
        o = att @ v
    else:
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    o = o.transpose(1, 2).contiguous().view(B, T, C)
    return F.linear(o, Wp.T, bp).numpy()


@pytest.mark.parametrize("manual", [False, True])
@pytest.mark.parametrize("B,T,C,H,bias", [(2, 33, 64, 4, True), (1, 1, 32, 1, True),
                                          (3, 17, 96, 3, False), (1, 64, 128, 2, True)])
def test_torch_reference(B, T, C, H, bias, manual):
    inp = make_inputs(B, T, C, H, bias=bias, dtype="f32", seed=7 + T, w_std=0.1,
                      proj_std=0.1)
    y = fwd(inp)["y"]
    yt = _torch_layer(inp, manual=manual)
    np.testing.assert_allclose(y, yt, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------- invariants I2 - I9
def test_rows_sum_to_one_and_future_is_zero():
    inp = tiny(B=2, T=12, C=16, H=4, w_std=1.0)
    P = fwd(inp, want=("P",))["P"]
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    T = P.shape[-1]
    upper = np.triu(np.ones((T, T), bool), k=1)
    assert np.all(P[..., upper] == 0.0)
    assert np.all(P[..., ~upper] > 0.0)      # diagonal and past are visible


def test_value_ones_gives_ones():
    """W_v = 0, b_v = 1 makes every value vector all-ones; with W_proj = I,
    b_proj = 0 the output equals the row sums of P, i.e. exactly 1."""
    B, T, C, H = 2, 20, 16, 4
    inp = tiny(B, T, C, H, w_std=0.7)
    inp.W_attn[:, 2 * C:] = 0.0
    inp.b_attn[2 * C:] = 1.0
    inp.W_proj[:] = np.eye(C, dtype=np.float32)
    inp.b_proj[:] = 0.0
    y = fwd(inp)["y"]
    np.testing.assert_allclose(y, 1.0, rtol=0, atol=1e-13)


def test_causality_bitwise():
    B, T, C, H = 2, 16, 32, 4
    inp = tiny(B, T, C, H, w_std=0.3)
    y0 = fwd(inp)["y"]
    rng = np.random.default_rng(5)
    for t in (0, 5, T - 2):
        pert = tiny(B, T, C, H, w_std=0.3)
        pert.x[:, t + 1:] += rng.standard_normal(pert.x[:, t + 1:].shape).astype(np.float32)
        y1 = fwd(pert)["y"]
        assert np.array_equal(y0[:, :t + 1], y1[:, :t + 1])
        assert not np.allclose(y0[:, t + 1:], y1[:, t + 1:])


def test_T1_is_cproj_of_v():
    B, C, H = 3, 32, 4
    inp = tiny(B, 1, C, H, w_std=0.3)
    y = fwd(inp)["y"]
    x = inp.x.astype(np.float64)[:, 0]
    v = x @ inp.W_attn[:, 2 * C:].astype(np.float64) + inp.b_attn[2 * C:]
    expect = v @ inp.W_proj.astype(np.float64) + inp.b_proj
    np.testing.assert_allclose(y[:, 0], expect, rtol=1e-13, atol=1e-14)


def test_constant_sequence():
    B, T, C, H = 2, 11, 16, 2
    inp = tiny(B, T, C, H, w_std=0.4)
    inp.x[:] = inp.x[:, :1]
    y = fwd(inp)["y"]
    y1 = fwd(inp.prefix(1))["y"]
    np.testing.assert_allclose(y, np.broadcast_to(y1, y.shape), rtol=1e-13, atol=1e-14)


def test_zero_query_gives_prefix_mean():
    B, T, C, H = 2, 13, 16, 4
    inp = tiny(B, T, C, H, w_std=0.4)
    inp.W_attn[:, :C] = 0.0
    inp.b_attn[:C] = 0.0
    o = fwd(inp, want=("ym", "qkv"))
    v = o["qkv"][:, :, 2 * C:]
    mean = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    np.testing.assert_allclose(o["ym"], mean, rtol=1e-12, atol=1e-14)


def test_prefix_permutation():
    B, T, C, H = 1, 10, 16, 2
    inp = tiny(B, T, C, H, w_std=0.5)
    y0 = fwd(inp)["y"]
    perm = np.random.default_rng(1).permutation(T - 1)
    inp.x[:, :T - 1] = inp.x[:, perm]
    y1 = fwd(inp)["y"]
    np.testing.assert_allclose(y1[:, T - 1], y0[:, T - 1], rtol=1e-12, atol=1e-14)


def test_head_permutation_and_batch_independence():
    B, T, C, H = 3, 9, 24, 3
    hs = C // H
    inp = tiny(B, T, C, H, w_std=0.5)
    y0 = fwd(inp)["y"]
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(p * hs, (p + 1) * hs) for p in perm])
    allcols = np.concatenate([cols, C + cols, 2 * C + cols])
    pinp = tiny(B, T, C, H, w_std=0.5)
    pinp.W_attn[:] = inp.W_attn[:, allcols]
    pinp.b_attn[:] = inp.b_attn[allcols]
    pinp.W_proj[:] = inp.W_proj[cols, :]
    y1 = fwd(pinp)["y"]
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-14)
    # batch independence: each sample alone gives the same rows, bitwise
    for b in range(B):
        yb = fwd(inp.batch(b, b + 1))["y"]
        assert np.array_equal(yb[0], y0[b])


def test_single_head_is_plain_attention():
    """H = 1: one head of size C; compare with a direct numpy formula."""
    B, T, C = 2, 8, 8
    inp = tiny(B, T, C, 1, w_std=0.5)
    o = fwd(inp, want=("ym", "qkv"))
    qkv = o["qkv"]
    for b in range(B):
        q, k, v = qkv[b, :, :C], qkv[b, :, C:2 * C], qkv[b, :, 2 * C:]
        s = q @ k.T / math.sqrt(C)
        s[np.triu(np.ones((T, T), bool), 1)] = -np.inf
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(o["ym"][b], p @ v, rtol=1e-12, atol=1e-14)


def test_empty_batch():
    inp = tiny(B=2, T=4, C=8, H=2)
    e = inp.batch(0, 0)
    assert fwd(e)["y"].shape == (0, 4, 8)


# ------------------------------------------------------------- backward
def _loss(inp, lib=None):
    return float((fwd(inp, lib=lib)["y"] * inp.dY.astype(np.float64)).sum())


def _fd_check(inp, n_per_tensor, rng, lib=None, eps=1e-6, tol=1e-6):
    g = oracle.backward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                        inp.dY, inp.n_head, lib=lib)
    # finite differences need fp64 inputs: work on float64 copies
    import dataclasses
    base = dataclasses.replace(
        inp, **{k: (None if getattr(inp, k) is None else getattr(inp, k).astype(np.float64))
                for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj", "dY")})
    worst = 0.0
    for name, gname in (("x", "dx"), ("W_attn", "dW_attn"), ("b_attn", "db_attn"),
                        ("W_proj", "dW_proj"), ("b_proj", "db_proj")):
        a = getattr(base, name)
        if a is None:
            continue
        flat = a.reshape(-1)
        for idx in rng.choice(flat.size, size=min(n_per_tensor, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + eps
            lp = _loss(base, lib)
            flat[idx] = old - eps
            lm = _loss(base, lib)
            flat[idx] = old
            fd = (lp - lm) / (2 * eps)
            an = g[gname].reshape(-1)[idx]
            err = abs(fd - an) / max(1.0, abs(an))
            worst = max(worst, err)
            assert err <= tol, (name, idx, fd, an)
    return worst


def test_backward_finite_differences_tiny():
    inp = make_inputs(2, 6, 8, 2, bias=True, dtype="f32", seed=3, w_std=0.5,
                      proj_std=0.5, with_dY=True)
    _fd_check(inp, 40, np.random.default_rng(0))


def test_backward_finite_differences_tiny_char_shape():
    """The tiny char workload's shape (B8 T64 C128 H4), 64 entries per tensor."""
    inp = workload_inputs(1, with_dY=True)
    _fd_check(inp, 64, np.random.default_rng(1))


def test_backward_matches_torch_autograd():
    import torch
    B, T, C, H = 2, 19, 32, 4
    inp = make_inputs(B, T, C, H, bias=True, dtype="f32", seed=11, w_std=0.2,
                      proj_std=0.2, with_dY=True)
    g = oracle.backward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                        inp.dY, H)
    ts = {k: torch.tensor(np.asarray(getattr(inp, k), np.float64), requires_grad=True)
          for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    import torch.nn.functional as F
    hs = C // H
    qkv = F.linear(ts["x"], ts["W_attn"].T, ts["b_attn"])
    q, k, v = [t.view(B, T, H, hs).transpose(1, 2) for t in qkv.split(C, 2)]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    y = F.linear(o.transpose(1, 2).reshape(B, T, C), ts["W_proj"].T, ts["b_proj"])
    y.backward(torch.from_numpy(inp.dY.astype(np.float64)))
    for k, gk in (("x", "dx"), ("W_attn", "dW_attn"), ("b_attn", "db_attn"),
                  ("W_proj", "dW_proj"), ("b_proj", "db_proj")):
        np.testing.assert_allclose(g[gk], ts[k].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_no_bias():
    inp = make_inputs(1, 5, 8, 2, bias=False, dtype="f32", seed=4, w_std=0.5,
                      proj_std=0.5, with_dY=True)
    g = oracle.backward(inp.x, inp.W_attn, None, inp.W_proj, None, inp.dY, 2)
    assert "db_attn" not in g and "db_proj" not in g
    _fd_check(inp, 20, np.random.default_rng(2))


def test_backward_causality():
    """An upstream gradient that is non-zero only at position t reaches the
    input only at positions <= t (the mask blocks every later position)."""
    B, T, C, H = 1, 8, 16, 2
    inp = make_inputs(B, T, C, H, bias=True, dtype="f32", seed=9, w_std=0.5,
                      proj_std=0.5, with_dY=True)
    t = 3
    inp.dY[:, :t] = 0.0
    inp.dY[:, t + 1:] = 0.0
    g = oracle.backward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                        inp.dY, H)
    assert np.all(g["dx"][:, t + 1:] == 0.0)
    assert np.any(g["dx"][:, :t] != 0.0)


# ----------------------------------------------------------- workloads
def test_workload_table():
    """Shapes of the named workloads and the c_proj init rule
    std = 0.02 / sqrt(2 * n_layer)."""
    assert WORKLOADS[2].proj_std == pytest.approx(0.02 / math.sqrt(24))
    assert WORKLOADS[2].proj_std == pytest.approx(0.0041, abs=5e-5)
    for i, w in WORKLOADS.items():
        assert w.C % w.H == 0
        assert w.hs in (32, 64)


def test_workload_prefix_is_causal_cut():
    """A ragged cut of the gpt2-xl-shape workload is a prefix of the full
    draw, so its output must be the prefix of the full output (bitwise)."""
    full = workload_inputs(4, B=1, T=40)
    cut = full.prefix(17)
    yf = fwd(full)["y"]
    yc = fwd(cut)["y"]
    assert np.array_equal(yf[:, :17], yc)


# ------------------------------------------------- bf16 storage emulation
def _bits_rne_bf16(a):
    """Round float64 values to bfloat16 (8 significant bits, nearest even)
    by integer arithmetic on the fp64 bit pattern: keep the top 7 explicit
    mantissa bits, i.e. drop the low 45 bits with round-half-even."""
    u = np.ascontiguousarray(a, np.float64).view(np.uint64)
    drop = np.uint64(45)
    half = np.uint64(1 << 44)
    lsb = (u >> drop) & np.uint64(1)
    r = ((u + half - np.uint64(1) + lsb) >> drop) << drop
    return r.view(np.float64)


def test_store_bf16_rounds_to_nearest_even():
    inp = make_inputs(2, 9, 32, 2, dtype="f32", seed=21, w_std=0.3, proj_std=0.3)
    exact = fwd(inp, want=("qkv", "ym"))
    r = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 2,
                       want=("qkv", "ym"), store_bf16=("qkv",))
    assert np.array_equal(r["qkv"], _bits_rne_bf16(exact["qkv"]))
    assert not np.array_equal(r["qkv"], exact["qkv"])
    r2 = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 2,
                        want=("ym",), store_bf16=("ym",))
    assert np.array_equal(r2["ym"], _bits_rne_bf16(exact["ym"]))
    # tie cases: exactly half-way values go to the even neighbour
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)])
    assert np.array_equal(_bits_rne_bf16(ties), [1.0, 1 + 2.0 ** -6, -1.0])


def test_store_bf16_is_identity_on_representable_values():
    """x in {-1, 0, 1}, weights in {0, +-1/2}, no bias: every q, k, v is a
    small multiple of 1/2, exactly representable in bf16, so rounding the
    stored qkv changes nothing (bitwise)."""
    rng = np.random.default_rng(3)
    B, T, C, H = 2, 8, 16, 2
    import dataclasses
    inp = make_inputs(B, T, C, H, bias=False, dtype="f32", seed=1)
    inp = dataclasses.replace(
        inp, x=rng.integers(-1, 2, (B, T, C)).astype(np.float32),
        W_attn=(rng.integers(-1, 2, (C, 3 * C)) * 0.5).astype(np.float32))
    a = fwd(inp)["y"]
    b = oracle.forward(inp.x, inp.W_attn, None, inp.W_proj, None, H,
                       store_bf16=("qkv",))["y"]
    assert np.array_equal(a, b)


def test_backward_store_bf16_rounds_exactly_the_stored_tensors():
    """Rounding a stored gradient changes nothing upstream of it, and the
    gradients downstream are the exact chain rule through the rounded
    values (checked with plain fp64 matrix products)."""
    B, T, C, H = 2, 9, 16, 2
    inp = make_inputs(B, T, C, H, dtype="f32", seed=12, w_std=0.4, proj_std=0.4, with_dY=True)
    args = (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, H)
    ex = oracle.backward(*args, want_inter=True)
    rd = oracle.backward(*args, want_inter=True, store_bf16=("dqkv",))
    assert np.array_equal(rd["dqkv"], _bits_rne_bf16(ex["dqkv"]))
    assert np.array_equal(rd["dym"], ex["dym"])
    x = inp.x.reshape(-1, C).astype(np.float64)
    g = rd["dqkv"].reshape(-1, 3 * C)
    np.testing.assert_allclose(rd["dW_attn"], x.T @ g, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rd["db_attn"], g.sum(0), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rd["dx"].reshape(-1, C), g @ inp.W_attn.T.astype(np.float64),
                               rtol=1e-12, atol=1e-13)
    r2 = oracle.backward(*args, want_inter=True, store_bf16=("dym",))
    assert np.array_equal(r2["dym"], _bits_rne_bf16(ex["dym"]))
    # stored merged heads: dW_proj = round(ym)^T dY
    r3 = oracle.backward(*args, store_bf16=("ym",))
    ym = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                        want=("ym",), store_bf16=("ym",))["ym"].reshape(-1, C)
    np.testing.assert_allclose(r3["dW_proj"], ym.T @ inp.dY.reshape(-1, C).astype(np.float64),
                               rtol=1e-12, atol=1e-13)
    # no rounding requested: bitwise the plain backward
    r4 = oracle.backward(*args, want_inter=True, store_bf16=())
    for k in ex:
        assert np.array_equal(r4[k], ex[k])


# --------------------------------- the bf16 path's P.V and dV weight rounding
def _constant_sequence(B, T, C, H, seed, **kw):
    """Inputs whose T positions all repeat position 0 of each sequence."""
    import dataclasses
    inp = make_inputs(B, T, C, H, dtype="f32", seed=seed, **kw)
    x = np.repeat(inp.x[:, :1], T, axis=1)
    dY = None if inp.dY is None else inp.dY
    return dataclasses.replace(inp, x=x, dY=dY)


def check_pv_weights_constant_sequence(lib=None):
    """Every score of a row is s = q.k / sqrt(hs), so the weights the bf16
    path feeds its P.V product are all u = 2^(t - ceil t) with t = s log2 e,
    each rounded to bf16, over n u: o_i = v bf16(u) / u for every i."""
    B, T, C, H = 2, 6, 16, 2
    hs = C // H
    inp = _constant_sequence(B, T, C, H, seed=41, w_std=0.6, b_attn_std=0.3)
    r = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                       want=("ym", "qkv"), store_bf16=("P",), lib=lib)
    qkv = r["qkv"]
    moved = 0
    for b in range(B):
        for h in range(H):
            q = qkv[b, 0, h * hs:(h + 1) * hs]
            k = qkv[b, 0, C + h * hs:C + (h + 1) * hs]
            v = qkv[b, 0, 2 * C + h * hs:2 * C + (h + 1) * hs]
            t = float(q @ k) / math.sqrt(hs) / math.log(2.0)
            assert abs(t - round(t)) > 1e-6  # the reference is unambiguous
            u = 2.0 ** (t - math.ceil(t))
            ratio = float(_bits_rne_bf16(np.array([u]))[0]) / u
            moved += ratio != 1.0
            for i in range(T):
                np.testing.assert_allclose(r["ym"][b, i, h * hs:(h + 1) * hs], v * ratio,
                                           rtol=1e-12, atol=1e-15)
    assert moved > 0


def check_value_grad_weights_constant_sequence(lib=None):
    """On a constant sequence p_ij = 1/(i+1) for j <= i, so with "Pb" the
    value gradient is dv_j = sum_{i>=j} bf16(1/(i+1)) dO_i; the query and
    key gradients are untouched."""
    B, T, C, H = 1, 7, 16, 2
    hs = C // H
    inp = _constant_sequence(B, T, C, H, seed=43, w_std=0.5, with_dY=True)
    args = (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, H)
    ex = oracle.backward(*args, want_inter=True, lib=lib)
    r = oracle.backward(*args, want_inter=True, store_bf16=("Pb",), lib=lib)
    w = _bits_rne_bf16(1.0 / np.arange(1, T + 1, dtype=np.float64))
    dO = ex["dym"][0]
    for h in range(H):
        want = np.array([(w[j:, None] * dO[j:, h * hs:(h + 1) * hs]).sum(0) for j in range(T)])
        np.testing.assert_allclose(r["dqkv"][0, :, 2 * C + h * hs:2 * C + (h + 1) * hs], want,
                                   rtol=1e-12, atol=1e-14)
    assert np.array_equal(r["dqkv"][..., :2 * C], ex["dqkv"][..., :2 * C])
    assert not np.array_equal(r["dqkv"][..., 2 * C:], ex["dqkv"][..., 2 * C:])


def test_pv_weights_constant_sequence():
    check_pv_weights_constant_sequence()


def test_value_grad_weights_constant_sequence():
    check_value_grad_weights_constant_sequence()


def test_pv_weights_error_bound_and_exact_outputs():
    """Each P.V weight moves by at most 2^-8 of itself (one rounding to 8
    significant bits), the normaliser is exact, so
    |o_P - o| <= 2^-8 sum_j p_ij |v_j|; the
    probabilities and log-sum-exp outputs are the exact softmax."""
    B, T, C, H = 2, 33, 32, 2
    hs = C // H
    inp = make_inputs(B, T, C, H, dtype="f32", seed=45, w_std=0.4, b_attn_std=0.2)
    ex = fwd(inp, want=("ym", "P", "lse", "qkv", "y"))
    r = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                       want=("ym", "P", "lse", "qkv"), store_bf16=("P",))
    assert np.array_equal(r["P"], ex["P"]) and np.array_equal(r["lse"], ex["lse"])
    assert np.array_equal(r["qkv"], ex["qkv"])
    v = np.abs(ex["qkv"][..., 2 * C:]).reshape(B, T, H, hs).transpose(0, 2, 1, 3)
    bound = (ex["P"] @ v).transpose(0, 2, 1, 3).reshape(B, T, C) * 2.0 ** -8
    err = np.abs(r["ym"] - ex["ym"])
    assert np.all(err <= bound * (1 + 1e-9) + 1e-15)
    assert err.max() > 0


def test_value_grad_weights_error_bound():
    """|dv_Pb - dv| <= 2^-8 sum_i p_ij |dO_i| (each weight rounded once)."""
    B, T, C, H = 2, 21, 32, 4
    hs = C // H
    inp = make_inputs(B, T, C, H, dtype="f32", seed=47, w_std=0.4, with_dY=True)
    args = (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, H)
    ex = oracle.backward(*args, want_inter=True)
    r = oracle.backward(*args, want_inter=True, store_bf16=("Pb",))
    P = fwd(inp, want=("P",))["P"]
    dO = np.abs(ex["dym"]).reshape(B, T, H, hs).transpose(0, 2, 1, 3)
    bound = (P.transpose(0, 1, 3, 2) @ dO).transpose(0, 2, 1, 3).reshape(B, T, C) * 2.0 ** -8
    err = np.abs(r["dqkv"][..., 2 * C:] - ex["dqkv"][..., 2 * C:])
    assert np.all(err <= bound * (1 + 1e-9) + 1e-15)
    assert err.max() > 0


def _softmax_grad_pieces(inp, fwd_store, lib=None):
    """Exact probabilities (pinned above), the oracle's merged heads and
    merged-head gradient for the numpy reassembly of the attention backward."""
    H = inp.n_head
    f = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                       want=("qkv", "ym", "P"), store_bf16=fwd_store, lib=lib)
    args = (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, H)
    return f, args


def _attn_grads_numpy(qkv, P, dO, o, H, row_from_o, round_ds):
    """dq, dk, dv of one sequence by matrix products over the whole T x T
    softmax (a different order of every sum than the oracle's loops)."""
    T, C3 = qkv.shape
    C = C3 // 3
    hs = C // H
    sc = 1.0 / math.sqrt(hs)
    dq, dk, dv = (np.zeros((T, C)) for _ in range(3))
    for h in range(H):
        s = slice(h * hs, (h + 1) * hs)
        q, k, v, g, p = qkv[:, s], qkv[:, C:][:, s], qkv[:, 2 * C:][:, s], dO[:, s], P[h]
        dp = g @ v.T
        D = (g * o[:, s]).sum(1) if row_from_o else (p * dp).sum(1)
        ds = np.tril(p * (dp - D[:, None]))
        if round_ds:
            ds = _bits_rne_bf16(ds)
        dq[:, s], dk[:, s], dv[:, s] = sc * ds @ k, sc * ds.T @ q, p.T @ g
    return np.concatenate([dq, dk, dv], 1)


def check_row_term_and_ds_rounding(lib=None):
    """"Do" takes the softmax gradient's row term from the stored merged
    heads, "dS" rounds dS to bf16 before the query and key gradients: both
    against a numpy reassembly from the exact probabilities; and with
    nothing rounded the row term from the merged heads is the Jacobian's
    row term (sum_j p_ij dp_ij = dO_i . o_i)."""
    B, T, C, H = 2, 11, 16, 2
    inp = make_inputs(B, T, C, H, dtype="f32", seed=49, w_std=0.5, proj_std=0.5,
                      with_dY=True)
    f, args = _softmax_grad_pieces(inp, ("qkv", "ym"), lib)
    ex = oracle.backward(*args, want_inter=True, lib=lib)
    plain_o = oracle.backward(*args, want_inter=True, store_bf16=("Do",), lib=lib)
    np.testing.assert_allclose(plain_o["dqkv"], ex["dqkv"], rtol=1e-10, atol=1e-13)
    r = oracle.backward(*args, want_inter=True, store_bf16=("qkv", "ym", "Do", "dS"), lib=lib)
    assert not np.allclose(r["dqkv"][..., :2 * C], ex["dqkv"][..., :2 * C], rtol=1e-6, atol=0)
    for b in range(B):
        want = _attn_grads_numpy(f["qkv"][b], f["P"][b], r["dym"][b], f["ym"][b], H,
                                 row_from_o=True, round_ds=True)
        np.testing.assert_allclose(r["dqkv"][b], want, rtol=1e-11, atol=1e-14)
    rs = oracle.backward(*args, want_inter=True, store_bf16=("dS",), lib=lib)
    fe, _ = _softmax_grad_pieces(inp, (), lib)
    for b in range(B):
        want = _attn_grads_numpy(fe["qkv"][b], fe["P"][b], ex["dym"][b], fe["ym"][b], H,
                                 row_from_o=False, round_ds=True)
        np.testing.assert_allclose(rs["dqkv"][b], want, rtol=1e-11, atol=1e-14)


def test_row_term_and_ds_rounding():
    check_row_term_and_ds_rounding()
