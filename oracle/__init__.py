"""Plain fp64 CPU oracle for the GPT-2 / nanoGPT causal self-attention layer.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It shares no code with the HIP library
(``gpt_causal_self_amd``) and imports nothing from it.

The arithmetic lives in ``oracle.c`` (double precision, written from the
definition on page "nanoGPT global flow", section 2.5 (B) CausalSelfAttention
and page "nanoGPT architecture explained step by step", section 3).  This
module only marshals numpy arrays into it.  ``brute.py`` holds a second,
pure-Python rendering of the same definition for tiny shapes.

Weights are taken as [in, out] (``y = x @ W + b``), the transpose of the
``nn.Linear`` storage.

Parity pins: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute force, library special cases, closed
forms, invariants, finite differences, planted-mistake checks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (portable -O2, no fast-math, so no sum
    is reassociated).  Returns the path of the shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-Wall",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _declare(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_forward.restype = i
    lib.oracle_forward.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp,
                                   dp, dp, dp, dp, i, i]
    lib.oracle_layernorm.restype = i
    lib.oracle_layernorm.argtypes = [i, i, dp, dp, dp, dp, i]
    lib.oracle_block_attn_forward.restype = i
    lib.oracle_block_attn_forward.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp,
                                              dp, i, i]
    lib.oracle_mlp_forward.restype = i
    lib.oracle_mlp_forward.argtypes = [i, i, i, dp, dp, dp, dp, dp, dp, dp, i, i]
    lib.oracle_backward.restype = i
    lib.oracle_backward.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp,
                                    dp, dp, dp, dp, dp, dp, dp, i, i]
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
    lib.oracle_dropout_threshold.restype = ctypes.c_uint32
    lib.oracle_dropout_threshold.argtypes = [ctypes.c_double]
    lib.oracle_dropout_threshold16.restype = ctypes.c_uint32
    lib.oracle_dropout_threshold16.argtypes = [ctypes.c_double]
    lib.oracle_dropout_keep_attn.restype = i
    lib.oracle_dropout_keep_attn.argtypes = [i, i, i, i, i, ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_dropout_keep_resid.restype = i
    lib.oracle_dropout_keep_resid.argtypes = [ctypes.c_long, i, ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_backward_dropout.restype = i
    lib.oracle_backward_dropout.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, ctypes.c_double,
                                            ctypes.c_uint64, dp, dp, dp, dp, dp, dp, dp, i, i]
    lib.oracle_forward_dropout.restype = i
    lib.oracle_forward_dropout.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, ctypes.c_double,
                                           ctypes.c_uint64, dp, dp, i, i]
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first if it is not there)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward(x, W_attn, b_attn, W_proj, b_proj, n_head, *, want=("y",),
            store_bf16=(), nthreads=None, lib=None):
    """Causal self-attention forward in fp64.

    x [B,T,C]; W_attn [C,3C]; b_attn [3C] or None; W_proj [C,C];
    b_proj [C] or None.  ``want`` selects outputs among
    "y" [B,T,C], "qkv" [B,T,3C], "ym" [B,T,C] (merged heads before c_proj),
    "P" [B,H,T,T] (attention probabilities), "lse" [B,H,T].
    ``store_bf16`` may name "qkv" and/or "ym": those intermediates are then
    rounded to bfloat16 (nearest-even) where a bf16 path stores them; all
    arithmetic stays fp64.  "P" forms the merged heads with the weights a
    bf16 path feeds its P.V product: each unnormalised weight, taken
    relative to a whole power of two, rounded to bfloat16, over the sum of
    the unrounded weights ("P" and "lse" outputs stay the exact softmax).
    Returns a dict of float64 arrays."""
    lib = lib or load()
    x = _f64(x)
    B, T, C = x.shape
    H = int(n_head)
    W_attn, b_attn, W_proj, b_proj = map(_f64, (W_attn, b_attn, W_proj, b_proj))
    assert W_attn.shape == (C, 3 * C) and W_proj.shape == (C, C)
    assert b_attn is None or b_attn.shape == (3 * C,)
    assert b_proj is None or b_proj.shape == (C,)
    out = {"y": np.empty((B, T, C))}
    if "qkv" in want:
        out["qkv"] = np.empty((B, T, 3 * C))
    if "ym" in want:
        out["ym"] = np.empty((B, T, C))
    if "P" in want:
        out["P"] = np.empty((B, H, T, T))
    if "lse" in want:
        out["lse"] = np.empty((B, H, T))
    rc = lib.oracle_forward(B, T, C, H, _ptr(x), _ptr(W_attn), _ptr(b_attn),
                            _ptr(W_proj), _ptr(b_proj), _ptr(out["y"]),
                            _ptr(out.get("qkv")), _ptr(out.get("ym")),
                            _ptr(out.get("P")), _ptr(out.get("lse")),
                            _fwd_bits(store_bf16), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_forward failed (bad shape or out of memory)")
    return {k: v for k, v in out.items() if k in want}


_STORE_BITS = {"qkv": 1, "ym": 2, "dym": 4, "dqkv": 8, "dyd": 16, "P": 32, "Pb": 64,
               "Do": 128, "dS": 256, "z32": 512}


def _fwd_bits(store_bf16):
    """Forward rounding options: "qkv", "ym", "P" (see ``forward``) and, for
    ``forward_dropout``, "z32" (the keep factor 1/(1-p) held as the nearest
    float)."""
    bad = set(store_bf16) - {"qkv", "ym", "P", "z32"}
    if bad:
        raise ValueError(f"unknown forward rounding option(s) {sorted(bad)}")
    return sum(_STORE_BITS[k] for k in set(store_bf16))


def backward(x, W_attn, b_attn, W_proj, b_proj, dY, n_head, *, want_inter=False,
             store_bf16=(), nthreads=None, lib=None, p=0.0, seed=0):
    """Exact fp64 gradient of the layer for upstream gradient dY [B,T,C].

    Returns dict with dx, dW_attn, dW_proj and (when the layer has biases)
    db_attn, db_proj; with ``want_inter`` also dqkv [B,T,3C] and dym.
    ``store_bf16`` may name "qkv", "ym", "dym", "dqkv" (and, with dropout,
    "dyd": the masked, rescaled upstream gradient of the c_proj output):
    those stored tensors are rounded to bfloat16 and the gradients are the
    exact chain rule through the rounded values.  "P" forms the forward's
    merged heads as ``forward`` does; "Pb" sums the value gradient over
    bf16(p_ij z_ij), the operand a bf16 path feeds that product (the softmax
    gradient itself uses the exact p); "Do" forms the softmax gradient's row
    term sum_j p_ij dp_ij as dO_i . o_i from the merged heads the forward
    stored; "dS" rounds each dS_ij to bfloat16 before the query and key
    gradients; with dropout "z32" holds the keep factor 1/(1-p) as the
    nearest float.  ``p`` > 0: gradient of the
    forward with dropout rate p and generator ``seed`` (forward_dropout)."""
    lib = lib or load()
    x = _f64(x)
    B, T, C = x.shape
    H = int(n_head)
    W_attn, b_attn, W_proj, b_proj, dY = map(_f64, (W_attn, b_attn, W_proj, b_proj, dY))
    assert dY.shape == x.shape
    out = {"dx": np.empty((B, T, C)), "dW_attn": np.empty((C, 3 * C)),
           "dW_proj": np.empty((C, C))}
    if b_attn is not None:
        out["db_attn"] = np.empty(3 * C)
    if b_proj is not None:
        out["db_proj"] = np.empty(C)
    if want_inter:
        out["dqkv"] = np.empty((B, T, 3 * C))
        out["dym"] = np.empty((B, T, C))
    bits = sum(_STORE_BITS[k] for k in set(store_bf16))
    args = (_ptr(out["dx"]), _ptr(out["dW_attn"]), _ptr(out.get("db_attn")),
            _ptr(out["dW_proj"]), _ptr(out.get("db_proj")), _ptr(out.get("dqkv")),
            _ptr(out.get("dym")), bits, int(nthreads or default_threads()))
    common = (B, T, C, H, _ptr(x), _ptr(W_attn), _ptr(b_attn), _ptr(W_proj), _ptr(b_proj),
              _ptr(dY))
    if p > 0:
        rc = lib.oracle_backward_dropout(*common, float(p), int(seed), *args)
    else:
        rc = lib.oracle_backward(*common, *args)
    if rc != 0:
        raise ValueError("oracle_backward failed (bad shape or out of memory)")
    return out


def layernorm(x, w, b, *, nthreads=None, lib=None):
    """LayerNorm over the last axis (biased variance, eps 1e-5), fp64."""
    lib = lib or load()
    x = _f64(x)
    C = x.shape[-1]
    out = np.empty_like(x)
    rc = lib.oracle_layernorm(int(x.size // C), C, _ptr(x), _ptr(_f64(w)), _ptr(_f64(b)),
                              _ptr(out), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_layernorm failed")
    return out


def block_attn_forward(x, ln_w, ln_b, W_attn, b_attn, W_proj, b_proj, n_head, *,
                       want_ln=False, store_bf16=(), nthreads=None, lib=None):
    """Attention half of a Pre-LN block: x + layer(ln_1(x)), fp64.
    ``store_bf16`` may name "ln", "qkv", "ym", "P"."""
    lib = lib or load()
    x = _f64(x)
    B, T, C = x.shape
    ln_w, ln_b, W_attn, b_attn, W_proj, b_proj = map(
        _f64, (ln_w, ln_b, W_attn, b_attn, W_proj, b_proj))
    out = np.empty((B, T, C))
    ln = np.empty((B, T, C)) if want_ln else None
    bits = _fwd_bits(set(store_bf16) - {"ln"}) | (16 if "ln" in store_bf16 else 0)
    rc = lib.oracle_block_attn_forward(B, T, C, int(n_head), _ptr(x), _ptr(ln_w), _ptr(ln_b),
                                       _ptr(W_attn), _ptr(b_attn), _ptr(W_proj), _ptr(b_proj),
                                       _ptr(out), _ptr(ln), bits,
                                       int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_block_attn_forward failed")
    return {"out": out, "ln": ln} if want_ln else {"out": out}


def mlp_forward(x, W_fc, b_fc, W_proj, b_proj, *, want_h=False, store_bf16=(),
                nthreads=None, lib=None):
    """MLP sublayer c_proj(gelu(c_fc(x))) in fp64; x [..., C]."""
    lib = lib or load()
    x = _f64(x)
    C = x.shape[-1]
    M = int(x.size // C)
    W_fc, b_fc, W_proj, b_proj = map(_f64, (W_fc, b_fc, W_proj, b_proj))
    F = W_fc.shape[1]
    assert W_fc.shape == (C, F) and W_proj.shape == (F, C)
    y = np.empty(x.shape)
    h = np.empty(x.shape[:-1] + (F,)) if want_h else None
    rc = lib.oracle_mlp_forward(M, C, F, _ptr(x), _ptr(W_fc), _ptr(b_fc), _ptr(W_proj),
                                _ptr(b_proj), _ptr(y), _ptr(h),
                                1 if "h" in store_bf16 else 0,
                                int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_mlp_forward failed")
    return {"y": y, "h": h} if want_h else {"y": y}


def philox4x32_10(ctr, key, *, lib=None):
    """Philox4x32-10 of a 4-word counter and a 2-word key -> 4 words."""
    lib = lib or load()
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib.oracle_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def dropout_threshold(p, *, lib=None):
    """Drop threshold of a 32-bit word (c_proj output stream)."""
    return int((lib or load()).oracle_dropout_threshold(float(p)))


def dropout_threshold16(p, *, lib=None):
    """Drop threshold of a 16-bit value (attention-weight stream)."""
    return int((lib or load()).oracle_dropout_threshold16(float(p)))


def dropout_keep_attn(b, h, H, i, j, p, seed, *, lib=None):
    lib = lib or load()
    return bool(lib.oracle_dropout_keep_attn(b, h, H, i, j, int(seed),
                                             lib.oracle_dropout_threshold16(float(p))))


def dropout_keep_resid(m, n, p, seed, *, lib=None):
    lib = lib or load()
    return bool(lib.oracle_dropout_keep_resid(m, n, int(seed),
                                              lib.oracle_dropout_threshold(float(p))))


def forward_dropout(x, W_attn, b_attn, W_proj, b_proj, n_head, p, seed, *, want_ym=False,
                    store_bf16=(), nthreads=None, lib=None):
    """Forward with dropout rate p on the attention weights and on the c_proj
    output (Philox masks keyed by ``seed``); fp64.  ``store_bf16`` may name
    "qkv", "ym" and "P" (as in ``forward``) and "z32" (the keep factor held
    as the nearest float)."""
    lib = lib or load()
    x = _f64(x)
    B, T, C = x.shape
    W_attn, b_attn, W_proj, b_proj = map(_f64, (W_attn, b_attn, W_proj, b_proj))
    y = np.empty((B, T, C))
    ym = np.empty((B, T, C)) if want_ym else None
    rc = lib.oracle_forward_dropout(
        B, T, C, int(n_head), _ptr(x), _ptr(W_attn), _ptr(b_attn), _ptr(W_proj), _ptr(b_proj),
        float(p), int(seed), _ptr(y), _ptr(ym), _fwd_bits(store_bf16),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_forward_dropout failed (bad arguments or out of memory)")
    out = {"y": y}
    if want_ym:
        out["ym"] = ym
    return out
