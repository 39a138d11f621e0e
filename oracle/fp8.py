"""Decoding of 8-bit floats (OCP FP8 E4M3) for the low-precision attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name quantisation as an inference optimisation to keep ("Scaling AI
inference across multiple GPUs using NVIDIA TensorRT with multi-device
inference support", opening section) but fix no format or recipe.  The reading
taken here: Q, K and V are given as E4M3 values with one f32 scale per tensor
(real value = decoded byte * scale), and the attention they define is the exact
attention of those real values -- the oracle's ordinary ``attention`` applied
to the decoded tensors.

E4M3 (OCP 8-bit float, the "fn" variant): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent 0 encodes subnormals m/8 * 2^-6; the two
codes with all exponent and mantissa bits set (0x7F, 0xFF) are NaN; there is no
infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode E4M3 bytes (any integer array) to float64; NaN for 0x7F / 0xFF."""
    b = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    out = sign * mag
    return np.where((b & 0x7F) == 0x7F, np.nan, out)
