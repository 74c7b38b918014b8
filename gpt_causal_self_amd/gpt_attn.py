"""Thin ctypes binding of ``libgpt_attn.so`` (C ABI in ``include/gpt_attn.h``,
``include/gpt_block.h`` and ``include/gpt_decode.h``).

Argument marshalling only: torch tensors supply device memory and
``torch.cuda.current_stream()`` supplies the stream; every step of the layer
runs in the library's HIP kernels.  The functions carry the C names.  If the
library has not been built this module raises on first use -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt_attn.so")

OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_OOM, ERR_HIP, ERR_STATE = range(8)
F32, BF16 = 0, 1

EXPORTED = ("gpt_attn_workspace_bytes", "gpt_attn_create", "gpt_attn_forward",
            "gpt_attn_backward", "gpt_attn_destroy", "gpt_attn_strerror",
            "gpt_attn_debug_workspace", "gpt_attn_set_stage_events",
            "gpt_attn_debug_backward", "gpt_layernorm", "gpt_attn_block_forward",
            "gpt_mlp_forward", "gpt_attn_decode", "gpt_attn_export_kv",
            "gpt_attn_set_dropout", "gpt_attn_forward_noalloc")

_lib = None


class GptAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {gpt_attn_strerror(code)} (status {code})")


def lib():
    """The loaded library; raises if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__; __graft_entry__.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.gpt_attn_workspace_bytes.argtypes = [i, i, i, i, i, ctypes.POINTER(sz)]
        L.gpt_attn_create.argtypes = [ctypes.POINTER(vp), i, i, i, i, i]
        L.gpt_attn_forward.argtypes = [vp, vp, i, i, vp, vp, vp, vp, i, vp, vp, i]
        L.gpt_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, vp]
        L.gpt_attn_destroy.argtypes = [vp]
        L.gpt_attn_set_stage_events.argtypes = [vp, ctypes.POINTER(vp), i]
        L.gpt_attn_strerror.argtypes = [i]
        L.gpt_attn_strerror.restype = ctypes.c_char_p
        L.gpt_attn_debug_workspace.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                               ctypes.POINTER(vp)]
        L.gpt_attn_debug_backward.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                              ctypes.POINTER(vp)]
        L.gpt_layernorm.argtypes = [vp, i, i, vp, vp, vp, vp]
        L.gpt_attn_block_forward.argtypes = [vp, vp, i, i, vp, vp, vp, vp, vp, vp, i, vp, vp]
        L.gpt_mlp_forward.argtypes = [vp, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gpt_attn_decode.argtypes = [vp, vp, i, i, vp, vp, vp, vp, i, vp, vp, i, vp, vp]
        L.gpt_attn_export_kv.argtypes = [vp, vp, vp, i, vp]
        L.gpt_attn_set_dropout.argtypes = [vp, ctypes.c_float, ctypes.c_ulonglong]
        L.gpt_attn_forward_noalloc.argtypes = [vp, i, i, i, i, vp, vp, vp, vp, vp, vp]
        for name in EXPORTED:
            if name != "gpt_attn_strerror":
                getattr(L, name).restype = i
        _lib = L
    return _lib


def _ptr(t):
    """Device pointer of a tensor (None -> NULL); raw ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != OK:
        raise GptAttnError(rc, where)


def gpt_attn_strerror(code: int) -> str:
    return lib().gpt_attn_strerror(int(code)).decode()


def gpt_attn_workspace_bytes(C, n_head, max_B, max_T, dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().gpt_attn_workspace_bytes(C, n_head, max_B, max_T, dtype,
                                          ctypes.byref(out)), "gpt_attn_workspace_bytes")
    return out.value


def gpt_attn_create(C, n_head, max_B, max_T, dtype) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().gpt_attn_create(ctypes.byref(h), C, n_head, max_B, max_T, dtype),
           "gpt_attn_create")
    return h


def gpt_attn_forward(h, x, W_attn, b_attn, W_proj, b_proj, n_head, y, stream=None,
                     save_for_backward=False, B=None, T=None):
    """x [B,T,C] -> y [B,T,C] (both preallocated device tensors)."""
    if B is None or T is None:
        B, T = int(x.shape[0]), int(x.shape[1])
    rc = lib().gpt_attn_forward(h, _ptr(x), B, T, _ptr(W_attn), _ptr(b_attn), _ptr(W_proj),
                                _ptr(b_proj), n_head, _ptr(y), _stream(stream),
                                1 if save_for_backward else 0)
    _check(rc, "gpt_attn_forward")


def gpt_attn_backward(h, x, W_attn, W_proj, dY, dx, dW_attn, db_attn, dW_proj, db_proj,
                      stream=None, B=None, T=None):
    if B is None or T is None:
        B, T = int(x.shape[0]), int(x.shape[1])
    rc = lib().gpt_attn_backward(h, _ptr(x), _ptr(W_attn), _ptr(W_proj), _ptr(dY), _ptr(dx),
                                 _ptr(dW_attn), _ptr(db_attn), _ptr(dW_proj), _ptr(db_proj),
                                 B, T, _stream(stream))
    _check(rc, "gpt_attn_backward")


NOALLOC_SCRATCH_BYTES = 80 << 20


def gpt_attn_forward_noalloc(x, W_attn, b_attn, W_proj, b_proj, n_head, y, stream=None,
                             B=None, T=None, C=None):
    """x [B,T,C] -> y [B,T,C] (bf16 device tensors) without a handle and
    without allocating: intermediates in the library's static scratch."""
    if B is None or T is None or C is None:
        B, T, C = int(x.shape[0]), int(x.shape[1]), int(x.shape[2])
    rc = lib().gpt_attn_forward_noalloc(_ptr(x), B, T, C, n_head, _ptr(W_attn), _ptr(b_attn),
                                        _ptr(W_proj), _ptr(b_proj), _ptr(y), _stream(stream))
    _check(rc, "gpt_attn_forward_noalloc")


def gpt_attn_set_dropout(h, p, seed):
    """Dropout rate p and Philox seed of the following forwards (p = 0: off)."""
    _check(lib().gpt_attn_set_dropout(h, float(p), int(seed) & 0xFFFFFFFFFFFFFFFF),
           "gpt_attn_set_dropout")


def gpt_attn_destroy(h):
    _check(lib().gpt_attn_destroy(h), "gpt_attn_destroy")


def gpt_attn_set_stage_events(h, events):
    """events: list of hipEvent_t handles (ints) or None to switch off."""
    if events is None:
        _check(lib().gpt_attn_set_stage_events(h, None, 0), "gpt_attn_set_stage_events")
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().gpt_attn_set_stage_events(h, arr, len(events)), "gpt_attn_set_stage_events")


def gpt_attn_debug_workspace(h):
    """(qkv, o, lse) device addresses of the workspace intermediates."""
    q, o, l = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().gpt_attn_debug_workspace(h, ctypes.byref(q), ctypes.byref(o), ctypes.byref(l)),
           "gpt_attn_debug_workspace")
    return q.value, o.value, l.value


def gpt_attn_debug_backward(h):
    """(dym, dqkv, delta) device addresses of the backward intermediates."""
    a, b, c = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().gpt_attn_debug_backward(h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "gpt_attn_debug_backward")
    return a.value, b.value, c.value


def gpt_layernorm(x, w, b, out, stream=None, M=None, C=None):
    """out = LayerNorm(x) over the last dimension (bf16 tensors)."""
    if M is None or C is None:
        C = int(x.shape[-1])
        M = int(x.numel() // C) if C else 0
    _check(lib().gpt_layernorm(_ptr(x), M, C, _ptr(w), _ptr(b), _ptr(out), _stream(stream)),
           "gpt_layernorm")


def gpt_attn_block_forward(h, x, ln_w, ln_b, W_attn, b_attn, W_proj, b_proj, n_head, out,
                           stream=None, B=None, T=None):
    """out = x + attn(ln_1(x)) on a bf16 handle."""
    if B is None or T is None:
        B, T = int(x.shape[0]), int(x.shape[1])
    rc = lib().gpt_attn_block_forward(h, _ptr(x), B, T, _ptr(ln_w), _ptr(ln_b), _ptr(W_attn),
                                      _ptr(b_attn), _ptr(W_proj), _ptr(b_proj), n_head,
                                      _ptr(out), _stream(stream))
    _check(rc, "gpt_attn_block_forward")


def gpt_mlp_forward(x, W_fc, b_fc, W_proj, b_proj, hbuf, y, residual=None, stream=None,
                    M=None, C=None, F=None):
    """y = gelu(x W_fc + b_fc) W_proj + b_proj (+ residual); hbuf receives the
    activations (bf16 tensors)."""
    if M is None or C is None or F is None:
        C = int(x.shape[-1])
        M = int(x.numel() // C) if C else 0
        F = int(W_fc.shape[-1])
    rc = lib().gpt_mlp_forward(_ptr(x), M, C, F, _ptr(W_fc), _ptr(b_fc), _ptr(W_proj),
                               _ptr(b_proj), _ptr(residual), _ptr(hbuf), _ptr(y),
                               _stream(stream))
    _check(rc, "gpt_mlp_forward")


def gpt_attn_decode(h, x_new, W_attn, b_attn, W_proj, b_proj, n_head, k_cache, v_cache, y,
                    pos, stream=None, B=None, cache_T=None):
    """One decode step at position pos: x_new [B, C] -> y [B, C]; k_cache and
    v_cache [B, H, cache_T, hs] receive this position's key and value."""
    if B is None:
        B = int(x_new.shape[0])
    if cache_T is None:
        cache_T = int(k_cache.shape[2])
    rc = lib().gpt_attn_decode(h, _ptr(x_new), B, pos, _ptr(W_attn), _ptr(b_attn), _ptr(W_proj),
                               _ptr(b_proj), n_head, _ptr(k_cache), _ptr(v_cache), cache_T,
                               _ptr(y), _stream(stream))
    _check(rc, "gpt_attn_decode")


def gpt_attn_export_kv(h, k_cache, v_cache, stream=None, cache_T=None):
    """Copy the keys and values of the last forward into the caches."""
    if cache_T is None:
        cache_T = int(k_cache.shape[2])
    _check(lib().gpt_attn_export_kv(h, _ptr(k_cache), _ptr(v_cache), cache_T, _stream(stream)),
           "gpt_attn_export_kv")


class Layer:
    """Owns one handle; allocates outputs with torch (plumbing only)."""

    def __init__(self, C, n_head, max_B, max_T, dtype="bf16"):
        self.C, self.n_head, self.max_B, self.max_T = C, n_head, max_B, max_T
        self.dtype = dtype
        self.h = gpt_attn_create(C, n_head, max_B, max_T, BF16 if dtype == "bf16" else F32)

    def forward(self, x, W_attn, b_attn, W_proj, b_proj, y=None, stream=None,
                save_for_backward=False):
        import torch
        if y is None:
            y = torch.empty_like(x)
        gpt_attn_forward(self.h, x, W_attn, b_attn, W_proj, b_proj, self.n_head, y,
                         stream=stream, save_for_backward=save_for_backward)
        return y

    def backward(self, x, W_attn, W_proj, dY, has_bias=True, stream=None):
        import torch
        dx = torch.empty_like(x)
        dW_attn = torch.empty_like(W_attn)
        dW_proj = torch.empty_like(W_proj)
        C = self.C
        db_attn = torch.empty(3 * C, dtype=x.dtype, device=x.device) if has_bias else None
        db_proj = torch.empty(C, dtype=x.dtype, device=x.device) if has_bias else None
        gpt_attn_backward(self.h, x, W_attn, W_proj, dY, dx, dW_attn, db_attn, dW_proj,
                          db_proj, stream=stream)
        out = {"dx": dx, "dW_attn": dW_attn, "dW_proj": dW_proj}
        if has_bias:
            out["db_attn"], out["db_proj"] = db_attn, db_proj
        return out

    def workspace(self, B, T):
        """Copies of the last forward's intermediates as torch tensors:
        q, k, v [B,H,T,hs], o [B,T,C], lse [B,H,T] (test access)."""
        import torch
        qa, oa, la = gpt_attn_debug_workspace(self.h)
        H, C = self.n_head, self.C
        hs = C // H
        td = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        qkv = torch.empty((3, B, H, T, hs), dtype=td, device="cuda")
        o = torch.empty((B, T, C), dtype=td, device="cuda")
        lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        _memcpy_d2d(qkv.data_ptr(), qa, qkv.numel() * qkv.element_size())
        _memcpy_d2d(o.data_ptr(), oa, o.numel() * o.element_size())
        _memcpy_d2d(lse.data_ptr(), la, lse.numel() * 4)
        return qkv, o, lse

    def backward_workspace(self, B, T):
        """Copies of the last backward's intermediates: dym [B,T,C],
        dqkv [B,T,3C], delta [B,H,T] (test access)."""
        import torch
        da, qa, la = gpt_attn_debug_backward(self.h)
        H, C = self.n_head, self.C
        td = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        dym = torch.empty((B, T, C), dtype=td, device="cuda")
        dqkv = torch.empty((B, T, 3 * C), dtype=td, device="cuda")
        delta = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        _memcpy_d2d(dym.data_ptr(), da, dym.numel() * dym.element_size())
        _memcpy_d2d(dqkv.data_ptr(), qa, dqkv.numel() * dqkv.element_size())
        _memcpy_d2d(delta.data_ptr(), la, delta.numel() * 4)
        return dym, dqkv, delta

    def close(self):
        if self.h is not None:
            gpt_attn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_hip = None


def _memcpy_d2d(dst: int, src: int, nbytes: int):
    """Synchronous device-to-device copy through the HIP runtime."""
    global _hip
    import torch
    torch.cuda.synchronize()
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    rc = _hip.hipMemcpy(ctypes.c_void_p(dst), ctypes.c_void_p(src), ctypes.c_size_t(nbytes), 3)
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")
