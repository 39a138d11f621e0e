"""fp64 reference for merging two partial attention results.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Ring Attention streams K/V chunks past the local queries and keeps an online
softmax, so each chunk c yields a partial result (O_c, LSE_c) over its own
keys ("Scaling AI inference across multiple GPUs using NVIDIA TensorRT with
multi-device inference support", section "Ring Attention").  For two disjoint
key sets a and b, the softmax over a U b splits as

  L = ln(e^La + e^Lb)                 computed as  M + ln(e^(La-M) + e^(Lb-M)),  M = max(La, Lb)
  O = e^(La-L) * Oa + e^(Lb-L) * Ob

which is exactly attention over the union (in real arithmetic).  A side with
no keys is (O = 0, LSE = -inf), the identity; two empty sides give
(O = 0, LSE = -inf), never NaN.

Pinned by tests/test_oracle.py: chunked-then-merged equals unchunked
attention, identity, commutativity, associativity.
"""
from __future__ import annotations

import numpy as np


def merge(o_a, lse_a, o_b, lse_b):
    """o_* [..., S, D], lse_* [..., S] -> (o, lse) in float64."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    if o_a.shape != o_b.shape or la.shape != lb.shape or o_a.shape[:-1] != la.shape:
        raise ValueError("merge operands must share shapes")
    m = np.maximum(la, lb)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    with np.errstate(invalid="ignore"):
        ea = np.exp(la - m_safe)          # exp(-inf) = 0 for an empty side
        eb = np.exp(lb - m_safe)
    tot = ea + eb
    lse = np.where(both_empty, -np.inf, m_safe + np.log(np.where(both_empty, 1.0, tot)))
    wa = np.where(both_empty, 0.0, ea / np.where(both_empty, 1.0, tot))
    wb = np.where(both_empty, 0.0, eb / np.where(both_empty, 1.0, tot))
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return o, lse
