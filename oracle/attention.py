"""fp64 reference for non-causal multi-head attention with per-row LSE.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed, per batch b and head h (all arithmetic in float64 on
the exact values of the stored inputs):

  z_ij  = scale * sum_d q_id k_jd                     (scaled scores)
  m_i   = max_j z_ij
  LSE_i = m_i + ln sum_j exp(z_ij - m_i)              (natural log)
  P_ij  = exp(z_ij - LSE_i)                           (softmax row, materialised)
  O_id  = sum_j P_ij v_jd

Sources: bidirectional (unmasked) attention of diffusion transformers, in
"Scaling AI inference across multiple GPUs using NVIDIA TensorRT with
multi-device inference support", section "Context parallelism"; the
QK^T -> Softmax -> times V chain with a total score scale of 1/sqrt(head_dim)
(split as a fourth root on each of Q and K) in "TensorRT multi-device
attention inference in practice", step 1.  The LSE output is not named on the
pages; it is the quantity Ring Attention's online softmax carries between K/V
chunks (section "Ring Attention" of the first page).

Empty key set (Skv = 0): the softmax has no terms, so LSE = ln 0 = -inf and O
is taken as 0, the identity of the partial-result merge.

Parity pins: tests/test_oracle.py.
"""
from __future__ import annotations

import numpy as np

_ROW_SUM_TOL = 1e-12


def _check(q, k, v):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return q, k, v


def _rows(qr: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Attention for a block of query rows of one (b, h): qr [r, D], k, v [Skv, D]."""
    r = qr.shape[0]
    if k.shape[0] == 0:
        return np.zeros((r, v.shape[1])), np.full(r, -np.inf)
    z = scale * (qr @ k.T)                       # [r, Skv] scaled scores
    m = z.max(axis=1)                            # row max
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    p = np.exp(z - lse[:, None])                 # the full softmax rows
    s = p.sum(axis=1)
    bad = np.abs(s - 1.0) > _ROW_SUM_TOL
    if np.any(bad & np.isfinite(s)):
        raise AssertionError(f"softmax rows do not sum to 1: worst {np.max(np.abs(s - 1.0))}")
    o = p @ v
    return o, lse


def attention(q, k, v, scale: float, row_block: int = 512):
    """Full attention.  q [B,H,Sq,D], k/v [B,H,Skv,D] -> O [B,H,Sq,D], LSE [B,H,Sq]."""
    q, k, v = _check(q, k, v)
    B, H, Sq, D = q.shape
    O = np.empty((B, H, Sq, v.shape[3]))
    L = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, row_block):
                r1 = min(Sq, r0 + row_block)
                O[b, h, r0:r1], L[b, h, r0:r1] = _rows(q[b, h, r0:r1], k[b, h], v[b, h], scale)
    return O, L


def attention_rows(q, k, v, scale: float, rows, row_block: int = 256):
    """Attention for a subset of query rows (same rows for every (b, h)).

    Returns O [B, H, len(rows), D] and LSE [B, H, len(rows)].
    """
    rows = np.asarray(rows, dtype=np.int64)
    qs = np.asarray(q)[:, :, rows, :]
    return attention(qs, k, v, scale, row_block=row_block)

