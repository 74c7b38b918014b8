"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/oracle.c``, plants one plausible mistake (a dropped
term, a wrong sign, a wrong index or offset, a transposed operand, a missing
scale or normalisation), compiles the copy into a temporary library and runs
a quick subset of the pins against it: brute-force loops, the T = 1 closed
form, torch fp64 autograd and finite differences.  Every mutant has to fail at
least one of them; the unmodified source has to pass all of them.  All of this
runs on the CPU; the oracle in the tree is never modified.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
import oracle.brute as brute
from gpt_causal_self_amd.inputs import make_inputs

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, [(old, new, occurrence index or None for every occurrence)])
MUTANTS = [
    ("bias dropped", [("row[n] += c->bias[n]", "row[n] += 0.0", 0)]),
    ("scale without sqrt", [("const double scale = 1.0 / sqrt((double)hs);",
                             "const double scale = 1.0 / (double)hs;", 0)]),
    ("future keys visible", [("for (int j = 0; j <= i; ++j)", "for (int j = 0; j < T; ++j)", k)
                             for k in (0, 0, 0, 0)]),
    ("diagonal masked", [("for (int j = 0; j <= i; ++j)", "for (int j = 0; j < i; ++j)", k)
                         for k in (0, 0, 0, 0)]),
    ("key read from value block",
     [("const double *k = qkv + ((size_t)b * T + j) * ld + C + (size_t)h * hs;",
       "const double *k = qkv + ((size_t)b * T + j) * ld + 2 * (size_t)C + (size_t)h * hs;", 0)]),
    ("query head offset dropped",
     [("const double *q = qkv + ((size_t)b * T + i) * ld + (size_t)h * hs;",
       "const double *q = qkv + ((size_t)b * T + i) * ld;", 0)]),
    ("heads merged in reverse order",
     [("double *o = c->ym + ((size_t)b * T + i) * C + (size_t)h * hs;",
       "double *o = c->ym + ((size_t)b * T + i) * C + (size_t)(H - 1 - h) * hs;", 0)]),
    ("softmax not normalised", [("p[j] /= Z;", "p[j] /= 1.0;", 0)]),
    ("exp argument negated", [("p[j] = exp(p[j] - m);", "p[j] = exp(m - p[j]);", 0)]),
    ("log-sum-exp loses max", [("return m + log(Z);", "return log(Z);", 0)]),
    ("square weight transposed",
     [("row[n] += a * w[n];",
       "row[n] += a * (c->K == c->N ? c->W[(size_t)n * c->N + k] : w[n]);", 0)]),
    ("softmax grad without row term",
     [("double ds = p[j] * (dp[j] - rowdot);", "double ds = p[j] * dp[j];", 0)]),
    ("key grad sign", [("dkj[d] += scale * ds * qi[d];", "dkj[d] -= scale * ds * qi[d];", 0)]),
    ("value grad wrong operand", [("dvj[d] += pv * dO[d];", "dvj[d] += pv * qi[d];", 0)]),
    ("query grad without scale", [("dqi[d] += scale * ds * kj[d];", "dqi[d] += ds * kj[d];", 0)]),
    ("bias grad drops last row",
     [("db[n] += dout[(size_t)m * N + n];",
       "db[n] += (m + 1 < M) ? dout[(size_t)m * N + n] : 0.0;", 0)]),
    ("weight grad drops first row",
     [("for (int m = 0; m < c->M; ++m) {", "for (int m = 1; m < c->M; ++m) {", 0)]),
    ("bf16 rounding keeps 7 bits", [("ldexp(nearbyint(ldexp(f, 8)), e - 8)",
                                     "ldexp(nearbyint(ldexp(f, 7)), e - 7)", 0)]),
    ("bf16 rounding truncates", [("ldexp(nearbyint(ldexp(f, 8)), e - 8)",
                                  "ldexp(trunc(ldexp(f, 8)), e - 8)", 0)]),
    ("layernorm unbiased variance", [("var /= c->C; /* biased", "var /= (c->C - 1); /* biased", 0)]),
    ("layernorm without eps", [("1.0 / sqrt(var + 1e-5)", "1.0 / sqrt(var)", 0)]),
    ("layernorm drops shift", [("+ (c->b ? c->b[i] : 0.0)", "+ 0.0", 0)]),
    ("gelu tanh approximation",
     [("return u * 0.5 * (1.0 + erf(u / sqrt(2.0)));",
       "return u * 0.5 * (1.0 + tanh(0.7978845608028654 * (u + 0.044715 * u * u * u)));", 0)]),
    ("block drops the residual", [("out[i] = x[i] + y[i];", "out[i] = y[i];", 0)]),
    ("mlp skips gelu", [("h[i] = gelu(h[i]);", "h[i] = h[i];", 0)]),
    ("philox multiplier", [("(uint64_t)0xD2511F53u * x0", "(uint64_t)0xD2511F57u * x0", 0)]),
    ("philox key schedule", [("k0 += 0x9E3779B9u;", "k0 += 0x9E3779B1u;", 0)]),
    ("dropout weights not rescaled", [("const double w = wp[j] * keep_scale;",
                                       "const double w = wp[j];", 0)]),
    ("residual dropout not rescaled", [("? y[(size_t)m * C + n] * keep_scale",
                                        "? y[(size_t)m * C + n]", 0)]),
    ("dropout word index", [("return w[c0 & 3] >= thresh;", "return w[0] >= thresh;", 0)]),
    ("attention dropout half", [("(w[(j & 7) >> 1] >> (16 * (j & 1))) & 0xFFFFu",
                                 "(w[(j & 7) >> 1]) & 0xFFFFu", 0)]),
    ("attention dropout group", [("{(uint32_t)j >> 3, (uint32_t)i", "{(uint32_t)j >> 2, (uint32_t)i", 0)]),
    ("dropout backward: value grad unmasked", [("double pv = p[j] * z;",
                                                "double pv = p[j];", 0)]),
    ("P.V weights relative to the exact max", [("const double M = ceil(tmax);",
                                                "const double M = tmax;", 0)]),
    ("P.V weights over the rounded sum", [("U += w[j];", "U += round_bf16(w[j]);", 0)]),
    ("P.V weights not rounded", [("w[j] = round_bf16(w[j]) / U;", "w[j] = w[j] / U;", 0)]),
    ("value-gradient weights not rounded", [("if (c->round_pb) pv = round_bf16(pv);", "", 0)]),
    ("dS not rounded", [("if (c->round_ds) ds = round_bf16(ds);", "", 0)]),
    ("keep factor not held as a float", [("return scale32 ? (double)(float)s : s;", "return s;", 0)]),
    ("row term from the merged heads uses the input",
     [("for (int d = 0; d < hs; ++d) rowdot += dO[d] * oi[d];",
       "for (int d = 0; d < hs; ++d) rowdot += dO[d] * qi[d];", 0)]),
    ("dropout backward: weight grad unmasked", [("dp[j] = s * z;", "dp[j] = s;", 0)]),
    ("dropout backward: output grad unmasked", [("? dY[(size_t)m * C + n] * ks", "? dY[(size_t)m * C + n]", 0)]),
    ("input grad with untransposed square weight",
     [("s += g[n] * w[n];",
       "s += g[n] * (c->K == c->N ? c->W[(size_t)n * c->N + k] : w[n]);", 0)]),
]


def _apply(src, edits):
    for old, new, occ in edits:
        parts = src.split(old)
        assert len(parts) > occ + 1, f"pattern not found: {old!r}"
        src = old.join(parts[:occ + 1]) + new + old.join(parts[occ + 1:])
    return src


def _pins(lib):
    """Quick subset of the oracle's pins; returns the names that failed."""
    failed = []
    # bf16 storage rounding against integer rounding of the fp64 bit pattern
    from test_oracle_pins import _bits_rne_bf16
    inp = make_inputs(2, 5, 16, 2, dtype="f32", seed=4, w_std=0.3, proj_std=0.3)
    ex = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 2,
                        want=("qkv",), lib=lib)["qkv"]
    rq = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 2,
                        want=("qkv",), store_bf16=("qkv",), lib=lib)["qkv"]
    if not np.array_equal(rq, _bits_rne_bf16(ex)):
        failed.append("bf16 rounding")
    # LayerNorm / MLP / block against torch fp64
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(9)
    xx = rng.standard_normal((6, 16)) * 2 + 1
    w16, b16 = 1 + 0.1 * rng.standard_normal(16), 0.1 * rng.standard_normal(16)
    T_ = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    if not np.allclose(oracle.layernorm(xx, w16, b16, lib=lib),
                       F.layer_norm(T_(xx), (16,), T_(w16), T_(b16), 1e-5).numpy(),
                       rtol=1e-12, atol=1e-12):
        failed.append("layernorm")
    Wf, Wp = rng.standard_normal((16, 64)) * 0.3, rng.standard_normal((64, 16)) * 0.3
    ym = oracle.mlp_forward(xx, Wf, None, Wp, None, lib=lib)["y"]
    if not np.allclose(ym, (F.gelu(T_(xx) @ T_(Wf)) @ T_(Wp)).numpy(), rtol=1e-11, atol=1e-13):
        failed.append("mlp")
    inb = make_inputs(1, 5, 16, 2, dtype="f32", seed=3, w_std=0.3, proj_std=0.3)
    ob = oracle.block_attn_forward(inb.x, w16, b16, inb.W_attn, inb.b_attn, inb.W_proj,
                                   inb.b_proj, 2, lib=lib)["out"]
    lnb = F.layer_norm(T_(inb.x), (16,), T_(w16), T_(b16), 1e-5).numpy()
    yb = oracle.forward(lnb, inb.W_attn, inb.b_attn, inb.W_proj, inb.b_proj, 2, lib=lib)["y"]
    if not np.allclose(ob, inb.x + yb, rtol=1e-12, atol=1e-13):
        failed.append("block")
    # dropout: Philox known answers, the element -> counter mapping, and the
    # composition against a numpy assembly of the pinned pieces
    import test_oracle_dropout_pins as dpin
    for ctr, key, want in dpin._kat():
        if oracle.philox4x32_10(ctr, key, lib=lib) != want:
            failed.append("philox kat")
            break
    thr, thr16 = oracle.dropout_threshold(0.5, lib=lib), oracle.dropout_threshold16(0.5, lib=lib)
    for (i, j) in ((3, 5), (7, 0), (9, 14), (2, 10), (4, 3), (8, 22)):
        w = oracle.philox4x32_10([j >> 3, i, 1 * 4 + 2, 1], [77, 0], lib=lib)
        u = (w[(j & 7) >> 1] >> (16 * (j & 1))) & 0xFFFF
        if oracle.dropout_keep_attn(1, 2, 4, i, j, 0.5, 77, lib=lib) != (u >= thr16):
            failed.append("dropout mapping")
            break
    for (m, n) in ((3, 5), (7, 0), (9, 14), (2, 10), (4, 3), (8, 22)):
        w = oracle.philox4x32_10([n >> 2, m, 0, 2], [77, 0], lib=lib)[n & 3]
        if oracle.dropout_keep_resid(m, n, 0.5, 77, lib=lib) != (w >= thr):
            failed.append("residual dropout mapping")
            break
    pd, sd = 0.5, 77
    di = make_inputs(1, 5, 8, 2, dtype="f32", seed=11, w_std=0.4, proj_std=0.4,
                     b_attn_std=0.2, b_proj_std=0.2)
    r = oracle.forward(di.x, di.W_attn, di.b_attn, di.W_proj, di.b_proj, 2,
                       want=("P", "qkv"), lib=lib)
    ymd = np.zeros((1, 5, 8))
    for h in range(2):
        Z = np.array([[oracle.dropout_keep_attn(0, h, 2, i, j, pd, sd, lib=lib)
                       for j in range(5)] for i in range(5)], dtype=float)
        ymd[0, :, 4 * h:4 * h + 4] = (r["P"][0, h] * Z / (1 - pd)) @ r["qkv"][0, :, 16 + 4 * h:20 + 4 * h]
    yd = ymd @ di.W_proj + di.b_proj
    Z2 = np.array([[oracle.dropout_keep_resid(t, n, pd, sd, lib=lib) for n in range(8)]
                   for t in range(5)], dtype=float)[None]
    yd = yd * Z2 / (1 - pd)
    got = oracle.forward_dropout(di.x, di.W_attn, di.b_attn, di.W_proj, di.b_proj, 2, pd, sd,
                                 lib=lib)["y"]
    if not np.allclose(got, yd, rtol=1e-12, atol=1e-14):
        failed.append("dropout composition")
    # dropout backward against central differences of the dropout forward
    dY = np.random.default_rng(5).standard_normal((1, 5, 8))
    A = {k: np.array(getattr(di, k), np.float64) for k in ("x", "W_attn", "W_proj")}
    gd = oracle.backward(A["x"], A["W_attn"], di.b_attn, A["W_proj"], di.b_proj, dY, 2,
                         p=pd, seed=sd, lib=lib)
    for k, gk in (("x", "dx"), ("W_attn", "dW_attn"), ("W_proj", "dW_proj")):
        flat = A[k].reshape(-1)
        for idx in (0, flat.size // 3, flat.size - 1):
            old = flat[idx]
            vals = []
            for e in (1e-6, -1e-6):
                flat[idx] = old + e
                yy = oracle.forward_dropout(A["x"], A["W_attn"], di.b_attn, A["W_proj"],
                                            di.b_proj, 2, pd, sd, lib=lib)["y"]
                vals.append(float(np.sum(yy * dY)))
            flat[idx] = old
            fd = (vals[0] - vals[1]) / 2e-6
            if abs(fd - gd[gk].reshape(-1)[idx]) > 1e-6 * max(1.0, abs(fd)):
                failed.append("dropout backward fd")
    # the bf16 path's P.V and value-gradient weights: closed forms on a
    # constant sequence
    import test_oracle_pins as opin
    try:
        opin.check_pv_weights_constant_sequence(lib)
    except AssertionError:
        failed.append("P.V weights closed form")
    try:
        opin.check_value_grad_weights_constant_sequence(lib)
    except AssertionError:
        failed.append("value-gradient weights closed form")
    try:
        opin.check_row_term_and_ds_rounding(lib)
    except AssertionError:
        failed.append("row term and dS rounding")
    try:
        dpin.check_single_precision_keep_factor(lib)
    except AssertionError:
        failed.append("single-precision keep factor")
    # brute force forward, incl. P and the log-sum-exp
    for (B, T, C, H, bias) in ((2, 5, 8, 2, True), (2, 6, 16, 4, False)):
        inp = make_inputs(B, T, C, H, bias=bias, dtype="f32", seed=T, w_std=0.5,
                          proj_std=0.5, b_attn_std=0.3, b_proj_std=0.3)
        try:
            o = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                               H, want=("y", "P", "lse", "qkv"), lib=lib)
        except Exception:
            failed.append("forward raised")
            continue
        yb, Pb = brute.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H)
        if not np.allclose(o["y"], yb, rtol=1e-12, atol=1e-13):
            failed.append("brute y")
        if not np.allclose(o["P"], Pb, rtol=1e-12, atol=1e-15):
            failed.append("brute P")
        qkv, hs = o["qkv"], C // H
        for b in range(B):
            for h in range(H):
                for i in range(T):
                    s = [float(qkv[b, i, h * hs:(h + 1) * hs] @
                               qkv[b, j, C + h * hs:C + (h + 1) * hs]) / math.sqrt(hs)
                         for j in range(i + 1)]
                    lse = math.log(sum(math.exp(v) for v in s))
                    if not abs(o["lse"][b, h, i] - lse) <= 1e-12 * max(1, abs(lse)):
                        failed.append("lse")
    # backward against torch fp64 autograd
    import torch
    import torch.nn.functional as F
    B, T, C, H = 2, 7, 16, 2
    hs = C // H
    inp = make_inputs(B, T, C, H, bias=True, dtype="f32", seed=2, w_std=0.4,
                      proj_std=0.4, with_dY=True)
    try:
        g = oracle.backward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj,
                            inp.dY, H, lib=lib)
    except Exception:
        failed.append("backward raised")
        return failed
    ts = {k: torch.tensor(np.asarray(getattr(inp, k), np.float64), requires_grad=True)
          for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    qkv = F.linear(ts["x"], ts["W_attn"].T, ts["b_attn"])
    q, k, v = [t.view(B, T, H, hs).transpose(1, 2) for t in qkv.split(C, 2)]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    y = F.linear(o.transpose(1, 2).reshape(B, T, C), ts["W_proj"].T, ts["b_proj"])
    y.backward(torch.from_numpy(inp.dY.astype(np.float64)))
    for kk, gk in (("x", "dx"), ("W_attn", "dW_attn"), ("b_attn", "db_attn"),
                   ("W_proj", "dW_proj"), ("b_proj", "db_proj")):
        if not np.allclose(g[gk], ts[kk].grad.numpy(), rtol=1e-10, atol=1e-12):
            failed.append("autograd " + gk)
    return failed


def test_unmodified_oracle_passes_quick_pins(tmp_path):
    out = str(tmp_path / "liboracle_same.so")
    oracle.build(SRC, out)
    assert _pins(oracle.load(out)) == []


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, edits):
    src = _apply(open(SRC).read(), edits)
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src)
    out = str(tmp_path / "liboracle_mutant.so")
    oracle.build(str(path), out)
    failed = _pins(oracle.load(out))
    assert failed, f"planted mistake '{name}' was not caught by any pin"
