"""Comparison rules shared by the GPU parity tests.

Readings of the tolerances (the design notes list them with their reasons):
  * "max relative error" is normwise: max_i |g_i - r_i| / max_i |r_i| over the
    compared tensor (elementwise relative error is unbounded near 0).
  * fp32 mode: normwise <= 1e-4 and exact argmax agreement on every row.
  * bf16 mode: normwise <= 2e-2 on logits and "admissible" argmax agreement
    >= 99.9%: a row agrees when the GPU's top token has an oracle logit within
    the logit tolerance (2e-2 * max|r|) of the oracle's top logit.  The exact
    agreement is always reported next to it.
  * argmax ties go to the lowest index on both sides (numpy convention).
"""
from __future__ import annotations

import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
ARGMAX_MIN = 0.999


def logits_report(gpu: np.ndarray, ref: np.ndarray, tol: float) -> dict:
    g = np.asarray(gpu, dtype=np.float64).reshape(-1, gpu.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    scale = np.abs(r).max()
    normwise = float(np.abs(g - r).max() / scale)
    ag, ar = g.argmax(-1), r.argmax(-1)
    exact = float((ag == ar).mean())
    r_top = r[np.arange(len(r)), ar]
    r_at_g = r[np.arange(len(r)), ag]
    admissible = float(((r_top - r_at_g) <= tol * scale).mean())
    floor = 1e-3 * scale
    big = np.abs(r) >= floor
    elem = float((np.abs(g - r)[big] / np.abs(r)[big]).max()) if big.any() else 0.0
    return {"normwise": normwise, "exact_argmax": exact, "admissible_argmax": admissible,
            "max_elem_rel_floor": elem, "rows": int(len(r)), "finite": bool(np.isfinite(g).all())}


def assert_logits(gpu, ref, dtype: str, label: str = "") -> dict:
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    rep = logits_report(gpu, ref, tol)
    print(f"[parity] {label} dtype={dtype} {rep}", flush=True)
    assert rep["finite"], f"{label}: non-finite GPU output"
    assert rep["normwise"] <= tol, f"{label}: normwise error {rep['normwise']:.3e} > {tol}"
    if dtype == "f32":
        assert rep["exact_argmax"] == 1.0, f"{label}: argmax disagreement in fp32 mode"
    else:
        assert rep["admissible_argmax"] >= ARGMAX_MIN, f"{label}: admissible argmax {rep['admissible_argmax']}"
    return rep


def normwise(gpu, ref) -> float:
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    return float(np.abs(g - r).max() / np.abs(r).max())
