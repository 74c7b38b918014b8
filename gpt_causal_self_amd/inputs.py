"""Seeded synthetic inputs for the causal self-attention layer.

This module holds only random draws, rounding to the storage dtype and the
named workload shapes; it contains none of the layer's arithmetic.  Both the
HIP path and the CPU oracle consume the same bytes produced here.

Recipe (one generator per workload, numpy PCG64 ``default_rng(123 + index)``;
the only seed the pages print is 123, page "GPT architecture: design ideas
and core concepts" (paozippq.com), demo code, model initialisation step):
  draw order x, W_attn, b_attn, W_proj, b_proj, dY, each as float32 standard
  normals times the workload's standard deviation; bf16 workloads then round
  every value to bfloat16 with round-to-nearest-even.

Standard deviations follow the pages' initialisation: N(0, 0.02) for the
linear layers (page "nanoGPT code analysis" (liaow.com), key design decisions
table, weight-initialisation row) and 0.02/sqrt(2*n_layer) for c_proj (page
"nanoGPT global flow walkthrough" (devpress.csdn.net), section 2.4).
x ~ N(0, 1) stands in for ln_1(x): LayerNorm output has zero mean and unit
variance per token.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_BASE = 123


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    T: int
    C: int
    H: int
    bias: bool
    dtype: str            # "f32" or "bf16"
    w_std: float          # W_attn
    b_attn_std: float
    proj_std: float       # W_proj
    b_proj_std: float
    backward: bool = False
    ragged_T: tuple = ()

    @property
    def hs(self) -> int:
        return self.C // self.H


WORKLOADS = {
    # block 64, batch 8, 4 heads, 128 embd (page "nanoGPT core code cheat sheet"
    # (pgsm.cn), section 6, memory-saving overrides)
    1: Workload(1, "tiny-char B8 T64 C128 H4 fp32", 8, 64, 128, 4, True, "f32",
                0.02, 0.02, 0.02 / math.sqrt(8), 0.0),
    # GPT-2 124M: batch 12, block 1024 (cheat sheet, section 4); 768/12 heads
    2: Workload(2, "gpt2-124M B12 T1024 C768 H12 bf16", 12, 1024, 768, 12, True,
                "bf16", 0.02, 0.02, 0.02 / math.sqrt(24), 0.02),
    # gpt2-medium shape (page "GPT architecture: design ideas and core concepts",
    # dynamic configuration section, GPT_CONFIGS)
    3: Workload(3, "gpt2-medium-shape B8 T1024 C1024 H16 bf16", 8, 1024, 1024,
                16, True, "bf16", 0.02, 0.02, 0.02 / math.sqrt(48), 0.02),
    # gpt2-xl shape, no bias, ragged sequence lengths
    4: Workload(4, "gpt2-xl-shape B4 T1024 C1600 H25 bf16 nobias", 4, 1024,
                1600, 25, False, "bf16", 0.02, 0.0, 0.02 / math.sqrt(96), 0.0,
                ragged_T=(1, 17, 128, 511, 1024)),
    # GPT-2 124M training step (forward + backward)
    5: Workload(5, "gpt2-124M fwd+bwd B12 T1024 C768 H12 bf16", 12, 1024, 768,
                12, True, "bf16", 0.02, 0.02, 0.02 / math.sqrt(24), 0.02,
                backward=True),
}


def round_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype; result is float32 holding
    exactly representable values."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return a.copy()
    if dtype == "bf16":
        return bf16_bits_to_f32(round_bf16_bits(a))
    raise ValueError(dtype)


@dataclasses.dataclass
class LayerInputs:
    dtype: str
    n_head: int
    x: np.ndarray
    W_attn: np.ndarray
    b_attn: np.ndarray | None
    W_proj: np.ndarray
    b_proj: np.ndarray | None
    dY: np.ndarray | None = None

    def prefix(self, T: int) -> "LayerInputs":
        """The same draws restricted to the first T positions."""
        return dataclasses.replace(
            self, x=np.ascontiguousarray(self.x[:, :T]),
            dY=None if self.dY is None else np.ascontiguousarray(self.dY[:, :T]))

    def batch(self, lo: int, hi: int) -> "LayerInputs":
        return dataclasses.replace(
            self, x=np.ascontiguousarray(self.x[lo:hi]),
            dY=None if self.dY is None else np.ascontiguousarray(self.dY[lo:hi]))


def make_inputs(B, T, C, H, *, bias=True, dtype="bf16", seed=SEED_BASE,
                w_std=0.02, b_attn_std=0.02, proj_std=0.02, b_proj_std=0.02,
                x_scale=1.0, qk_std=None, with_dY=False) -> LayerInputs:
    """Draw one set of layer inputs.  ``qk_std`` (optional) redraws the q and
    k column blocks of W_attn with a larger deviation to sharpen the softmax;
    ``x_scale`` multiplies x.  Both are stress knobs for tests."""
    rng = np.random.default_rng(seed)
    f32 = np.float32

    def normal(shape, std):
        return rng.standard_normal(shape, dtype=np.float32) * f32(std)

    x = normal((B, T, C), 1.0) * f32(x_scale)
    W_attn = normal((C, 3 * C), w_std)
    b_attn = normal((3 * C,), b_attn_std) if bias else None
    W_proj = normal((C, C), proj_std)
    if bias:
        b_proj = normal((C,), b_proj_std) if b_proj_std > 0 else np.zeros(C, np.float32)
    else:
        b_proj = None
    dY = normal((B, T, C), 1.0) if with_dY else None
    if qk_std is not None:
        W_attn[:, :2 * C] = normal((C, 2 * C), qk_std)
    rd = lambda a: None if a is None else to_dtype(a, dtype)  # noqa: E731
    return LayerInputs(dtype, H, rd(x), rd(W_attn), rd(b_attn), rd(W_proj),
                       rd(b_proj), rd(dY))


def workload_inputs(index: int, *, B=None, T=None, with_dY=None) -> LayerInputs:
    """Inputs of a named workload (optionally with a smaller batch or
    sequence: the draws are made at full size and then cut, so a cut is a
    prefix of the full workload)."""
    w = WORKLOADS[index]
    inp = make_inputs(w.B, w.T, w.C, w.H, bias=w.bias, dtype=w.dtype,
                      seed=SEED_BASE + index, w_std=w.w_std,
                      b_attn_std=w.b_attn_std, proj_std=w.proj_std,
                      b_proj_std=w.b_proj_std,
                      with_dY=w.backward if with_dY is None else with_dY)
    if T is not None and T != w.T:
        inp = inp.prefix(T)
    if B is not None and B != w.B:
        inp = inp.batch(0, B)
    return inp


def make_ln_params(C, *, seed, dtype="bf16", w_std=0.1, b_std=0.1, bias=True):
    """LayerNorm weight and bias.  GPT-2 initialises them to 1 and 0; the
    tests draw them around that point (1 + N(0, w_std), N(0, b_std)) so that
    a swapped or dropped scale or shift is visible."""
    rng = np.random.default_rng(seed)
    w = 1.0 + rng.standard_normal(C, dtype=np.float32) * np.float32(w_std)
    b = rng.standard_normal(C, dtype=np.float32) * np.float32(b_std) if bias else None
    return to_dtype(w, dtype), None if b is None else to_dtype(b, dtype)


@dataclasses.dataclass
class MlpInputs:
    x: np.ndarray            # [M, C]
    W_fc: np.ndarray         # [C, F]
    b_fc: np.ndarray | None  # [F]
    W_proj: np.ndarray       # [F, C]
    b_proj: np.ndarray | None
    residual: np.ndarray | None


def make_mlp_inputs(M, C, F, *, seed, dtype="bf16", bias=True, with_residual=False,
                    w_std=0.02, proj_std=0.02 / math.sqrt(24), b_std=0.02):
    """MLP sublayer inputs: x ~ N(0, 1) standing in for ln_2(x); c_fc weights
    N(0, 0.02) and the residual projection N(0, 0.02 / sqrt(2 n_layer)) as the
    pages' initialisation (n_layer = 12 by default); draw order x, W_fc, b_fc,
    W_proj, b_proj, residual."""
    rng = np.random.default_rng(seed)
    f32 = np.float32

    def normal(shape, std):
        return rng.standard_normal(shape, dtype=np.float32) * f32(std)

    x = normal((M, C), 1.0)
    W_fc = normal((C, F), w_std)
    b_fc = normal((F,), b_std) if bias else None
    W_proj = normal((F, C), proj_std)
    b_proj = normal((C,), b_std) if bias else None
    res = normal((M, C), 1.0) if with_residual else None
    rd = lambda a: None if a is None else to_dtype(a, dtype)  # noqa: E731
    return MlpInputs(rd(x), rd(W_fc), rd(b_fc), rd(W_proj), rd(b_proj), rd(res))


def to_torch(a: np.ndarray | None, dtype: str, device="cpu"):
    """Host float32 array (already representable in ``dtype``) -> torch
    tensor of that dtype on ``device``; bf16 goes through its bit pattern so
    no rounding happens on the way."""
    import torch
    if a is None:
        return None
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    bits = round_bf16_bits(a)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def from_torch(t) -> np.ndarray:
    """torch tensor (any float dtype, any device) -> float64 numpy, exact."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
