"""CPU checks of the C ABI: the library loads, exports every function that
``include/gpt_attn.h``, ``include/gpt_block.h`` and ``include/gpt_decode.h``
declare, and its host-only paths (argument
validation, workspace sizing, status strings) behave as documented.  No
compute call is made here."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from gpt_causal_self_amd import gpt_attn as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in ("gpt_attn.h", "gpt_block.h", "gpt_decode.h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"^(?:const char \*|int )\s*(gpt_\w+)\s*\(", text, re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ga.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ga.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert set(names) == set(ga.EXPORTED), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_strerror_covers_every_code(lib):
    seen = set()
    for code in range(8):
        s = ga.gpt_attn_strerror(code)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in ga.gpt_attn_strerror(99)


@pytest.mark.parametrize("args,code", [
    ((768, 12, 12, 1024, ga.BF16), ga.OK),
    ((0, 12, 12, 1024, ga.BF16), ga.ERR_INVALID_ARG),
    ((768, 0, 12, 1024, ga.BF16), ga.ERR_INVALID_ARG),
    ((768, 12, 0, 1024, ga.BF16), ga.ERR_INVALID_ARG),
    ((768, 12, 12, -1, ga.BF16), ga.ERR_INVALID_ARG),
    ((768, 12, 12, 1024, 7), ga.ERR_INVALID_ARG),
    ((770, 12, 12, 1024, ga.BF16), ga.ERR_SHAPE),
    ((1536, 12, 12, 1024, ga.BF16), ga.ERR_UNSUPPORTED),   # hs = 128
    ((192, 12, 12, 1024, ga.BF16), ga.ERR_UNSUPPORTED),    # hs = 16
    ((128, 4, 8, 64, ga.F32), ga.OK),
])
def test_workspace_bytes_validation(lib, args, code):
    out = ctypes.c_size_t(0)
    rc = lib.gpt_attn_workspace_bytes(*args, ctypes.byref(out))
    assert rc == code
    if code == ga.OK:
        C, H, B, T, dt = args
        es = 2 if dt == ga.BF16 else 4
        # at least q/k/v + merged heads + log-sum-exp
        assert out.value >= (4 * B * T * C) * es + B * H * T * 4


def test_create_validates_before_touching_the_device(lib):
    h = ctypes.c_void_p(123)
    assert lib.gpt_attn_create(ctypes.byref(h), 770, 12, 1, 1, ga.BF16) == ga.ERR_SHAPE
    assert h.value is None                      # *out cleared on error
    assert lib.gpt_attn_create(None, 768, 12, 1, 1, ga.BF16) == ga.ERR_INVALID_ARG
    assert lib.gpt_attn_create(ctypes.byref(h), 768, 12, 1, 1, 5) == ga.ERR_INVALID_ARG


def test_null_handle_paths(lib):
    assert lib.gpt_attn_destroy(None) == ga.OK
    assert lib.gpt_attn_forward(None, None, 1, 1, None, None, None, None, 1, None, None, 0) \
        == ga.ERR_INVALID_ARG
    assert lib.gpt_attn_backward(None, None, None, None, None, None, None, None, None, None,
                                 1, 1, None) == ga.ERR_INVALID_ARG
    assert lib.gpt_attn_debug_workspace(None, None, None, None) == ga.ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ga, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ga, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        ga.lib()


def test_block_entry_points_validate_on_the_host(lib):
    """Argument errors of the Block entry points return before any device
    call (no GPU here)."""
    p = ctypes.c_void_p(4096)      # aligned, never dereferenced
    odd = ctypes.c_void_p(4098)    # not 16-byte aligned
    L = lib
    assert L.gpt_layernorm(None, 4, 64, p, p, p, None) == ga.ERR_INVALID_ARG
    assert L.gpt_layernorm(p, -1, 64, p, p, p, None) == ga.ERR_INVALID_ARG
    assert L.gpt_layernorm(p, 4, 0, p, p, p, None) == ga.ERR_INVALID_ARG
    assert L.gpt_layernorm(p, 4, 60, p, p, p, None) == ga.ERR_SHAPE
    assert L.gpt_layernorm(p, 4, 8200, p, p, p, None) == ga.ERR_SHAPE
    assert L.gpt_layernorm(odd, 4, 64, p, p, p, None) == ga.ERR_ALIGN
    assert L.gpt_layernorm(p, 0, 64, p, None, p, None) == ga.OK       # empty: no-op
    assert L.gpt_mlp_forward(p, 4, 64, 256, None, p, p, p, None, p, p, None) == ga.ERR_INVALID_ARG
    assert L.gpt_mlp_forward(p, 4, 64, 250, p, p, p, p, None, p, p, None) == ga.ERR_SHAPE
    assert L.gpt_mlp_forward(p, 4, 64, 256, p, p, p, p, odd, p, p, None) == ga.ERR_ALIGN
    assert L.gpt_mlp_forward(p, 0, 64, 256, p, None, p, None, None, p, p, None) == ga.OK
    assert L.gpt_attn_block_forward(None, p, 1, 1, p, p, p, p, p, p, 4, p, None) \
        == ga.ERR_INVALID_ARG


def test_decode_entry_points_validate_on_the_host(lib):
    p = ctypes.c_void_p(4096)
    L = lib
    assert L.gpt_attn_decode(None, p, 1, 0, p, p, p, p, 4, p, p, 8, p, None) == ga.ERR_INVALID_ARG
    assert L.gpt_attn_export_kv(None, p, p, 8, None) == ga.ERR_INVALID_ARG
