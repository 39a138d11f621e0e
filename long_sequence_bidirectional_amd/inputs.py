"""Seeded synthetic inputs shared by the tests, the bench and the oracle's checks.

This module only draws random numbers and stores them in the two storage
types the library reads (fp32, and bf16 as raw 16-bit words).  It holds none
of the attention, merge or relayout arithmetic, so the CPU oracle and the HIP
path can both be fed from it without sharing any part of the computation.

Workload shapes model the Cosmos 3 video workload described in "Simplifying
model serving across multiple GPUs with TensorRT multi-device integration in
Dynamo-Triton" (section on distributing Cosmos 3 with Ulysses context
parallelism): 44160 video tokens, 5520 tokens per rank at a context-parallel
degree of 8, and a replicated 2992-token text path.  Head count 24 and head
dim 128 are an assumption (the pages do not state them).

Recipe: one ``numpy.random.SeedSequence(seed)`` spawns independent PCG64
streams; each tensor is i.i.d. N(0, 1) drawn as float32 and rounded to bf16
with round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import functools
from dataclasses import dataclass

import numpy as np

SEED = 42

# Stream indices of SeedSequence(SEED).spawn(N_STREAMS) (child i depends only on i).
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_KT, _STREAM_VT, _STREAM_SMALL = range(6)
_STREAM_P4_Q, _STREAM_P4_K, _STREAM_P4_V, _STREAM_P4_W = range(6, 10)
N_STREAMS = 10

# Shapes of the attention sample of "TensorRT multi-device attention inference in practice"
# (its single-device run: sequence length 56320, batch 1; 32 heads of 128, fp16; two ranks).
P4_SEQ = 56320
P4_HEADS = 32
P4_RANKS = 2

# Global shapes of the video workload (see module docstring).
S_VIDEO = 44160
S_TEXT = 2992
N_HEADS = 24
HEAD_DIM = 128
CP_DEGREE = 8
S_LOCAL = S_VIDEO // CP_DEGREE  # 5520 tokens per rank


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  Inputs here are finite
    normal draws, so NaN handling is not needed and is not attempted.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(stream: int, seed: int = SEED) -> np.random.Generator:
    ss = np.random.SeedSequence(seed).spawn(N_STREAMS)[stream]
    return np.random.Generator(np.random.PCG64(ss))


def normal_f32(shape, rng: np.random.Generator, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def normal_bf16(shape, rng: np.random.Generator, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) draws stored as bf16 bit patterns (uint16)."""
    return f32_to_bf16_bits(normal_f32(shape, rng, scale))


@functools.lru_cache(maxsize=2)
def video_set(seed: int = SEED, S: int = S_VIDEO, H: int = N_HEADS, D: int = HEAD_DIM,
              S_text: int = S_TEXT):
    """The one global tensor set every bf16 workload slices.

    Returns a dict of bf16 bit arrays: ``q``, ``k``, ``v`` of shape
    [1, H, S, D] and ``k_text``, ``v_text`` of shape [1, H, S_text, D].
    Arrays are read-only so cached copies cannot be modified by callers.
    """
    out = {
        "q": normal_bf16((1, H, S, D), _rng(_STREAM_Q, seed)),
        "k": normal_bf16((1, H, S, D), _rng(_STREAM_K, seed)),
        "v": normal_bf16((1, H, S, D), _rng(_STREAM_V, seed)),
        "k_text": normal_bf16((1, H, S_text, D), _rng(_STREAM_KT, seed)),
        "v_text": normal_bf16((1, H, S_text, D), _rng(_STREAM_VT, seed)),
    }
    for a in out.values():
        a.setflags(write=False)
    return out


def small_f32_set(B=1, H=2, S=256, D=64, seed: int = SEED):
    """The tiny fp32 self-attention case: q, k, v float32 [B, H, S, D]."""
    rng = _rng(_STREAM_SMALL, seed)
    q = normal_f32((B, H, S, D), rng)
    k = normal_f32((B, H, S, D), rng)
    v = normal_f32((B, H, S, D), rng)
    return q, k, v


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP FP8 E4M3 codes (nearest, ties to even; magnitudes above 448
    saturate to 448).  Returns uint8 codes.  Finite inputs only.

    Works on the float32 bit pattern: normal E4M3 values keep 3 of float32's 23 mantissa bits;
    below 2^-6 the spacing is fixed at 2^-9, which is handled by rounding x * 2^9 to an
    integer (exact in float32 for these magnitudes).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    sign = (x.view(np.uint32) >> np.uint32(31)).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(x), np.float32(448.0))
    bits = a.view(np.uint32)
    # normal range: round the float32 mantissa to 3 bits (ties to even), rebias 127 -> 7
    lsb = (bits >> np.uint32(20)) & np.uint32(1)
    r = (bits + np.uint32(0x7FFFF) + lsb) >> np.uint32(20)          # [exp8 | mant3]
    e = (r >> np.uint32(3)).astype(np.int64) - 127 + 7
    normal = ((e << 3) | (r & np.uint32(7)).astype(np.int64)).astype(np.int64)
    # subnormal range (|x| < 2^-6 before rounding): multiples of 2^-9
    sub = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)       # 0..8 (8 = smallest normal)
    code = np.where(a < np.float32(2.0 ** -6), sub, normal)
    return (code.astype(np.uint8) | sign)


def normal_e4m3(shape, rng: np.random.Generator, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) draws stored as E4M3 codes (uint8)."""
    return f32_to_e4m3(normal_f32(shape, rng, scale))


def random_e4m3(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    return normal_e4m3(shape, np.random.Generator(np.random.PCG64(seed)), scale)


def normal_f16(shape, rng: np.random.Generator, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) draws stored as IEEE fp16 (float32 draws rounded to nearest even)."""
    return normal_f32(shape, rng, scale).astype(np.float16)


def random_f16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    return normal_f16(shape, np.random.Generator(np.random.PCG64(seed)), scale)


@functools.lru_cache(maxsize=1)
def p4_set(seed: int = SEED, S: int = P4_SEQ, H: int = P4_HEADS, D: int = HEAD_DIM):
    """Inputs of the attention sample's single-device run: fp16 q, k, v in its
    (seq, batch, heads, head_dim) order with batch 1, i.e. [1, S, H, D], and the two
    RMSNorm weights w_q, w_k [D] (fp16).  All i.i.d. N(0, 1); read-only arrays."""
    rw = _rng(_STREAM_P4_W, seed)
    out = {
        "q": normal_f16((1, S, H, D), _rng(_STREAM_P4_Q, seed)),
        "k": normal_f16((1, S, H, D), _rng(_STREAM_P4_K, seed)),
        "v": normal_f16((1, S, H, D), _rng(_STREAM_P4_V, seed)),
        "w_q": normal_f16((D,), rw),
        "w_k": normal_f16((D,), rw),
    }
    for a in out.values():
        a.setflags(write=False)
    return out


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Independent seeded bf16 tensor for ad-hoc test shapes."""
    return normal_bf16(shape, np.random.Generator(np.random.PCG64(seed)), scale)


def random_f32(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    return normal_f32(shape, np.random.Generator(np.random.PCG64(seed)), scale)


@dataclass(frozen=True)
class Workload:
    """One named workload: which slices of the global set feed attention."""
    name: str
    description: str


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "fp32 self-attention B=1 H=2 S=256 D=64, scale 1/8"),
    "ulysses_rank": Workload("ulysses_rank", "bf16 self-attention H=3 S=44160 D=128 (one rank's "
                             "head subset at CP degree 8) plus pack/unpack of a [5520,24,128] shard"),
    "allgather_kv_rank": Workload("allgather_kv_rank", "bf16 attention Q 5520 rows vs K/V 44160 rows, "
                                  "H=24 D=128"),
    "ring_rank": Workload("ring_rank", "bf16 Q 5520 rows vs 8 K/V chunks of 5520 rows, H=24 D=128, "
                          "per-chunk partials merged by LSE"),
    "video_layer": Workload("video_layer", "bf16 self-attention S=44160 H=24 D=128 plus cross-attention "
                            "to 2992 text tokens, 36 times (one denoising step's layers)"),
    "p4_sample": Workload("p4_sample", "fp16 QK-RMSNorm prologue + attention, sequence-major [1,56320,32,128]: "
                          "the single-device run, and one rank of two under AllGather-KV (28160 query rows)"),
}


def sample_rows(S: int, n_random: int = 64, seed: int = SEED, extra=()) -> np.ndarray:
    """Row indices for sampled checks at full size.

    Fixed rows cross 128- and 256-row tile edges, the 5520-token shard edge
    and the ragged tail; the rest are seeded random rows.
    """
    fixed = [0, 1, 127, 128, 255, 256, 5503, 5504, 5519, 5520, S - 129, S - 128, S - 2, S - 1]
    fixed.extend(extra)
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    rnd = rng.integers(0, S, size=n_random)
    rows = np.unique(np.array([r for r in fixed if 0 <= r < S] + list(rnd), dtype=np.int64))
    return rows
