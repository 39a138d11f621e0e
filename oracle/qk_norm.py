"""fp64 reference of the QK-RMSNorm prologue of the attention sample.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "TensorRT multi-device attention inference in practice", step 1 (the
single-device model).  After the Q/K/V projections are reshaped to
(seq, batch, heads, head_dim), Q and K each go through an RMSNorm over
head_dim evaluated in fp32,

    y_d = x_d / sqrt(mean_d(x_d^2) + eps) * w_d,      eps = 1e-6,

with a weight vector w, and are cast back to fp16; then each is multiplied by
the fourth root of 1/head_dim, the 1/sqrt(head_dim) score scale split over Q
and K, before QK^T -> softmax -> times V.

Readings (the page names the steps and the fp32/fp16 casts, nothing finer):
- w is one head_dim-long vector per tensor (one for Q, one for K), stored in
  the model's 16-bit type;
- the norm and the weight product are evaluated exactly here (float64) and
  rounded once, to the 16-bit type, at the cast the page names.  An fp32
  evaluation differs from the exact value by a few fp32 ulps, which changes
  the rounded result only for values that close to a rounding boundary;
- the split scale is itself a 16-bit constant, and the product of two 16-bit
  values is rounded once to the 16-bit type (exact products of two 16-bit
  values fit in float64, so this step has no reading to choose).

The same prologue in bf16 uses the same steps with bf16 rounding.

Parity pins: tests/test_oracle.py.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x, w, eps: float) -> np.ndarray:
    """Exact RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w, in float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if w.shape != (x.shape[-1],):
        raise ValueError(f"weight shape {w.shape} does not match the last axis of {x.shape}")
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def round_to_f16(x) -> np.ndarray:
    """float64 -> IEEE binary16, round to nearest, ties to even (numpy's direct conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 value (returned as float64), round to nearest, ties to even.

    Directly from the float64 value (no pass through float32): the significand
    is scaled to 8 bits and rounded with numpy's rint (ties to even).  Finite
    normal inputs only, which is all the prologue produces.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _round(x, dtype: str):
    if dtype == "f16":
        return round_to_f16(x).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown 16-bit type {dtype!r}")


def qk_prologue(x, w, eps: float = 1e-6, post_scale: float | None = None, dtype: str = "f16") -> np.ndarray:
    """The prologue of one of Q or K: the 16-bit RMSNorm output, then (optionally) times
    the 16-bit constant post_scale, each result rounded to the 16-bit type.

    x holds the stored 16-bit input values, w the stored 16-bit weights (any float
    dtype holding those exact values).  Returns the 16-bit results as float64.
    """
    y = _round(rms_norm(x, w, eps), dtype)
    if post_scale is not None:
        s = float(_round(np.float64(post_scale), dtype))
        y = _round(y * s, dtype)
    return y
