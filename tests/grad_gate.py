"""Gates for the bf16 gradients of the training step.

The stated bf16 tolerance, |g - r| <= 2e-2 + 1e-2 |r| elementwise, is held
against the oracle run with the roundings that the bf16 path's precision
fixes, each applied in fp64 at the point where the path applies it:

  "qkv", "ym"   the stored q/k/v and merged heads (forward),
  "P"           the softmax weights fed to the P.V product (forward),
  "dym", "dqkv" the stored gradients of the merged heads and of qkv,
  "Pb"          the weights fed to the value-gradient product (backward),
  "Do"          the softmax gradient's row term sum_j p_ij dP_ij formed as
                dO_i . o_i from the stored merged heads (backward),
  "dS"          the dS operand of the query and key gradient products,
  "dyd"         with dropout: the stored masked, rescaled upstream gradient,
  "z32"         with dropout: the keep factor 1/(1-p), held as a float.

Against that oracle the path's remaining differences are its fp32 sums and
the final rounding of each gradient.  On top of it the normwise gate
||g - r|| / ||r|| <= 1e-2 holds against the exact oracle (no rounding at
all)."""
from __future__ import annotations

import numpy as np

import oracle

STORE = ("qkv", "P", "ym", "dym", "Pb", "Do", "dS", "dqkv")
GRADS = ("dx", "dW_attn", "db_attn", "dW_proj", "db_proj")
ATOL, RTOL, NORMWISE = 2e-2, 1e-2, 1e-2


def references(inp, p=0.0, seed=0):
    """(exact, rounded) oracle gradients of the layer for ``inp`` (bf16
    inputs with dY), optionally through dropout masks of rate p."""
    args = (inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.dY, inp.n_head)
    store = STORE + (("dyd", "z32") if p > 0 else ())
    exact = oracle.backward(*args, p=p, seed=seed)
    emul = oracle.backward(*args, p=p, seed=seed, store_bf16=store)
    return exact, emul


def check(name, g, r_emul, r_exact):
    """Elementwise stated gate against the rounding oracle, normwise gate
    against the exact one.  Returns (max err / bound, normwise error)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r_emul, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), name
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    if not np.all(err <= bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{name}: {(err > bound).sum()} / {err.size} out of the stated "
                             f"gate; worst at {i}: got {g[i]!r} want {r[i]!r} "
                             f"(bound {bound[i]:.3e})")
    x = np.asarray(r_exact, np.float64)
    rel = np.linalg.norm(g - x) / max(np.linalg.norm(x), 1e-30)
    assert rel <= NORMWISE, f"{name}: normwise relative error {rel:.3e} against the exact oracle"
    return float((err / bound).max()), float(rel)


def check_all(g, inp, p=0.0, seed=0):
    exact, emul = references(inp, p, seed)
    out = {}
    for k in GRADS:
        if k not in exact:
            assert g.get(k) is None, k
            continue
        out[k] = check(k, g[k], emul[k], exact[k])
    return out
