"""Reference index maps for the DeepSpeed Ulysses sequence<->head relayout.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Ulysses starts with the sequence split across P ranks; an all-to-all on Q, K
and V gives every rank the whole sequence for a disjoint subset of heads, and
a second all-to-all returns the attention output to the sequence split
("Scaling AI inference across multiple GPUs using NVIDIA TensorRT with
multi-device inference support", section "DeepSpeed Ulysses"; the Cosmos 3
setting of 5520 tokens per rank at degree 8 in "Simplifying model serving
across multiple GPUs with NVIDIA TensorRT multi-device integration in NVIDIA
Dynamo-Triton", section on distributing Cosmos 3 with Ulysses).

Readings (the pages give no layouts): rank r owns tokens
[r*S_l, (r+1)*S_l) and heads [r*Hp, (r+1)*Hp) with Hp = H/P; a shard is
token-major [B, S_l, H, D]; a send/receive buffer is [B, P, S_l, Hp, D] whose
chunk p goes to (or came from) rank p.

  seq->head pack    dst[b,p,s,h,d]      = src[b,s,p*Hp+h,d]      [B,S_l,H,D]   -> [B,P,S_l,Hp,D]
  seq->head unpack  dst[b,h,p*S_l+s,d]  = src[b,p,s,h,d]         [B,P,S_l,Hp,D] -> [B,Hp,P*S_l,D]
  head->seq pack    dst[b,p,s,h,d]      = src[b,h,p*S_l+s,d]     [B,Hp,P*S_l,D] -> [B,P,S_l,Hp,D]
  head->seq unpack  dst[b,s,g*Hp+h,d]   = src[b,g,s,h,d]         [B,P,S_l,Hp,D] -> [B,S_l,H,D]

Each map is written as a numpy reshape + transpose; the result is unique, so
comparisons against it are bit-exact.  Pinned by explicit index loops,
bijection and round-trip checks in tests/test_oracle.py.
"""
from __future__ import annotations

import numpy as np

SEQ_TO_HEAD = 0
HEAD_TO_SEQ = 1


def ulysses_pack(src: np.ndarray, P: int, direction: int) -> np.ndarray:
    src = np.asarray(src)
    if direction == SEQ_TO_HEAD:
        B, S_l, H, D = src.shape
        if H % P:
            raise ValueError("H must be divisible by P")
        return np.ascontiguousarray(src.reshape(B, S_l, P, H // P, D).transpose(0, 2, 1, 3, 4))
    if direction == HEAD_TO_SEQ:
        B, Hp, S, D = src.shape
        if S % P:
            raise ValueError("sequence must be divisible by P")
        return np.ascontiguousarray(src.reshape(B, Hp, P, S // P, D).transpose(0, 2, 3, 1, 4))
    raise ValueError("bad direction")


def ulysses_unpack(src: np.ndarray, P: int, direction: int) -> np.ndarray:
    src = np.asarray(src)
    B, P_, S_l, Hp, D = src.shape
    if P_ != P:
        raise ValueError("leading chunk dim must equal P")
    if direction == SEQ_TO_HEAD:
        return np.ascontiguousarray(src.transpose(0, 3, 1, 2, 4).reshape(B, Hp, P * S_l, D))
    if direction == HEAD_TO_SEQ:
        return np.ascontiguousarray(src.transpose(0, 2, 1, 3, 4).reshape(B, S_l, P * Hp, D))
    raise ValueError("bad direction")


def alltoall(send_bufs):
    """Simulated all-to-all over P ranks held in one address space.

    ``send_bufs[p]`` is rank p's send buffer [B, P, ...] (chunk r goes to rank
    r).  Returns ``recv[r]`` with chunk p = ``send_bufs[p][:, r]``.
    """
    P = len(send_bufs)
    return [np.ascontiguousarray(np.stack([send_bufs[p][:, r] for p in range(P)], axis=1))
            for r in range(P)]
