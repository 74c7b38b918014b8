"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

``oracle.c`` is compiled with gcc's address and undefined-behaviour
sanitizers (no recovery: the first finding aborts) and loaded into a fresh
Python process with the sanitizer runtime preloaded.  That process runs the
brute-force, finite-difference and autograd pins and every rounding option
against the sanitized library, so an out-of-bounds access, a use after free
or undefined arithmetic anywhere on those paths ends the run.  CPU only."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import math, sys
import numpy as np
sys.path.insert(0, ROOT); sys.path.insert(0, os.path.join(ROOT, "tests"))
import oracle, oracle.brute as brute
from gpt_causal_self_amd.inputs import make_inputs
import test_oracle_pins as pins
import test_oracle_dropout_pins as dpins
lib = oracle.load(LIB)
# brute force: forward, P and the log-sum-exp
for (B, T, C, H, bias) in ((2, 5, 8, 2, True), (1, 9, 16, 4, False), (2, 1, 8, 1, True)):
    inp = make_inputs(B, T, C, H, bias=bias, dtype="f32", seed=T, w_std=0.5, proj_std=0.5)
    o = oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H,
                       want=("y", "P", "lse", "qkv", "ym"), lib=lib)
    yb, Pb = brute.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, H)
    assert np.allclose(o["y"], yb, rtol=1e-12, atol=1e-13)
    assert np.allclose(o["P"], Pb, rtol=1e-12, atol=1e-15)
# finite differences of the backward (tiny shape and the tiny char shape, sampled)
rng = np.random.default_rng(0)
pins._fd_check(pins.tiny(with_dY=True), 6, rng, lib=lib)
# every rounding option, plain and with dropout, block, MLP, LayerNorm
inp = make_inputs(2, 13, 16, 2, dtype="bf16", seed=3, w_std=0.4, with_dY=True)
args = (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, 2)
every = ("qkv", "P", "ym", "dym", "Pb", "Do", "dS", "dqkv")
oracle.backward(*args, store_bf16=every, lib=lib)
oracle.backward(*args, store_bf16=every + ("dyd", "z32"), p=0.3, seed=9, lib=lib)
oracle.forward_dropout(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 2, 0.3, 9,
                       want_ym=True, store_bf16=("qkv", "P", "ym", "z32"), lib=lib)
w, b = np.ones(16), np.zeros(16)
oracle.block_attn_forward(inp.x, w, b, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, 2,
                          want_ln=True, store_bf16=("ln", "qkv", "P", "ym"), lib=lib)
oracle.mlp_forward(inp.x, np.ones((16, 32)) * 0.1, None, np.ones((32, 16)) * 0.1, None,
                   want_h=True, store_bf16=("h",), lib=lib)
pins.check_pv_weights_constant_sequence(lib)
pins.check_value_grad_weights_constant_sequence(lib)
pins.check_row_term_and_ds_rounding(lib)
dpins.check_single_precision_keep_factor(lib)
# empty batch
oracle.forward(np.zeros((0, 4, 8)), inp.W_attn[:8, :24], None, inp.W_proj[:8, :8], None, 2,
               lib=lib)
print("SANITIZED_OK")
'''


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not asan or not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
                    "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-fast-math", "-ffp-contract=off", src, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="1")
    code = f"import os\nROOT = {ROOT!r}\nLIB = {lib!r}\n" + SCRIPT
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "SANITIZED_OK" in r.stdout, (
        f"sanitized oracle run failed (rc {r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}")
