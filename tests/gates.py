"""Tolerance gates shared by the mutation tests and the GPU parity tests.

Attention output (against the fp64 oracle): max-abs <= 2e-2 and mean-abs <= 2e-3
over every compared element, plus relative L2 <= 1e-2.

Prologue output (bf16 Q', K' against the fp64 oracle), per element:
|gpu - ref| <= 2**-8 * (|ref| + 1).  The relative term is the worst case of one
round-to-nearest to bf16 (half an ulp is at most 2**-8 of the value); the
absolute term covers the fp32 evaluation, chiefly the fp32 rotary angle
pos * w_j whose error grows with the position (<= ~2e-4 rad at |pos| < 2**11,
times |y| <= ~8).  Plus mean-abs <= 2e-3 over all elements.
"""
from __future__ import annotations

import numpy as np

ATT_MAX_ABS = 2e-2
ATT_MEAN_ABS = 2e-3
ATT_REL_L2 = 1e-2
PRO_REL = 2.0 ** -8
PRO_ABS = 2.0 ** -8
PRO_MEAN_ABS = 2e-3


def attention_errors(out: np.ndarray, ref: np.ndarray) -> dict:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(out - ref)
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "rel_l2": float(np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-300)),
        "finite": bool(np.all(np.isfinite(out))),
    }


def attention_ok(out, ref) -> tuple[bool, dict]:
    e = attention_errors(out, ref)
    ok = (e["finite"] and e["max_abs"] <= ATT_MAX_ABS and e["mean_abs"] <= ATT_MEAN_ABS
          and e["rel_l2"] <= ATT_REL_L2)
    return ok, e


def prologue_errors(out: np.ndarray, ref: np.ndarray) -> dict:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(out - ref)
    bound = PRO_REL * np.abs(ref) + PRO_ABS
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "worst_ratio": float((d / bound).max()) if d.size else 0.0,
        "finite": bool(np.all(np.isfinite(out))),
    }


def prologue_ok(out, ref) -> tuple[bool, dict]:
    e = prologue_errors(out, ref)
    ok = e["finite"] and e["worst_ratio"] <= 1.0 and e["mean_abs"] <= PRO_MEAN_ABS
    return ok, e


# Gradients (backward pass), bf16 dq/dk/dv against the fp64 oracle.  Each
# gradient is a sum of products whose bf16 operands (P, dS and the output) carry
# a relative rounding of at most 2**-9 each, and dS = P (dP - delta) can cancel,
# so the error is bounded relative to the tensor's scale rather than to each
# element: relative L2 <= 1e-2 (about 2.5 times the 2**-8 of two such roundings)
# and max-abs <= 2**-6 of the tensor's largest magnitude.  The fp32 gamma
# gradients are sums over every row with fp32 accumulation: max-abs <= 1e-3 of
# the largest magnitude.
GRAD_REL_L2 = 1e-2
GRAD_MAX_REL = 2.0 ** -6
DGAMMA_MAX_REL = 1e-3


def gradient_errors(out, ref) -> dict:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(out - ref)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "max_over_scale": float(d.max() / max(scale, 1e-300)) if d.size else 0.0,
        "rel_l2": float(np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-300)),
        "finite": bool(np.all(np.isfinite(out))),
    }


def gradient_ok(out, ref) -> tuple[bool, dict]:
    e = gradient_errors(out, ref)
    return e["finite"] and e["rel_l2"] <= GRAD_REL_L2 and e["max_over_scale"] <= GRAD_MAX_REL, e


def dgamma_ok(out, ref) -> tuple[bool, dict]:
    e = gradient_errors(out, ref)
    return e["finite"] and e["max_over_scale"] <= DGAMMA_MAX_REL, e
