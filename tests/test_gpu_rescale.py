"""GPU parity of the online softmax's running-max raise with a nonzero O.

The 16-bit attention kernel keeps a running max m per query row and raises it
only when a key block's max exceeds it by more than 2^8 (base 2); then O and
the row sum are multiplied by alpha = 2^(m_old - m_new) before the block is
added (the online softmax of Ring Attention's blockwise streaming: "Scaling AI
inference across multiple GPUs using NVIDIA TensorRT with multi-device
inference support", section "Ring Attention").  With N(0,1) inputs at scale
1/sqrt(D) no block after the first ever triggers that raise, so these cases
plant it.

Construction: every query row has q[0] = 8 and every ordinary key k[0] = 0, so
dimension 0 adds nothing to ordinary scores.  A planted key has k[0] = beta and
zeros elsewhere, so its score is exactly delta = 8 * beta * scale for every
row:
- "dominant": one key with delta ~ 30 (natural units): the raise fires and that
  key takes essentially all of the weight;
- "moderate": one key with delta ~ 9.5: the raise fires for almost every row
  (the first block's max would have to exceed 3.95), yet the keys before it
  keep ~10% of the weight, so a wrong alpha on O or on the row sum shows up in
  O well beyond the gates;
- "block": every key of one block raised by delta ~ 8 on top of its own random
  score: a raise with a whole block of comparable new weights.
Placements in a 1000-key set (16 blocks of 64, the last one 40 keys): block 5
(inside the check-free steady-state loop when unsplit), block 14 (a full block
in the final per-block steps) and the ragged last block 15.  With a workspace
the planner splits each 256-row tile into four key pieces of four blocks, so
the planted block sits inside a piece, after that piece's first block.

Gates: the required ones (O max-abs 2e-2, mean-abs 2e-3) and the diagnostics of
helpers.assert_bf16_parity (bf16) or the fp16 ones (rel-L2 2e-3, LSE 1e-4).
Their derivation for these cases: the weight of the key that set m is exactly
2^0 = 1 (no rounding), every other weight is rounded to the 16-bit type with a
relative error of at most u (2^-9 bf16, 2^-12 fp16), and O is rounded once more
(u relative); so |dO| <= 2 u max|v| ~ 1.7e-2 for bf16 and ~2e-3 for fp16 at
max|v| ~ 4.3, and the mean error is near u |O|.  The LSE depends only on f32
scores (relative error ~1e-7 of |score| <= 40).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import assert_bf16_parity, dev_bf16, f64_of_bf16, host64, log, scale_of

B, H, SQ, SKV, D = 1, 2, 300, 1000, 128
PLACEMENT_BLOCK = {"steady": 5, "late": 14, "ragged": 15}
KIND_DELTA = {"dominant": 30.0, "moderate": 9.5, "block": 8.0}
F16_REL_L2 = 2e-3
F16_LSE_MAX_ABS = 1e-4


def _to16(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> the stored 16-bit array (bf16 bit patterns or float16)."""
    x = np.asarray(x, np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float16)


def _f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return f64_of_bf16(a) if dtype == "bf16" else a.astype(np.float64)


@functools.lru_cache(maxsize=None)
def case_data(kind: str, placement: str, dtype: str):
    """Stored 16-bit q, k, v and the oracle's (O, LSE) of the planted case."""
    seed = 8100 + 10 * list(KIND_DELTA).index(kind) + list(PLACEMENT_BLOCK).index(placement)
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, H, SQ, D)).astype(np.float32)
    k = g.standard_normal((B, H, SKV, D)).astype(np.float32)
    v = g.standard_normal((B, H, SKV, D)).astype(np.float32)
    scale = scale_of(D)
    q[..., 0] = 8.0
    k[..., 0] = 0.0
    blk = PLACEMENT_BLOCK[placement]
    beta = KIND_DELTA[kind] / (8.0 * scale)
    if kind == "block":
        lo, hi = blk * 64, min(SKV, blk * 64 + 64)
        k[:, :, lo:hi, 0] = beta
    else:
        j = min(SKV - 1, blk * 64 + 29)        # the ragged block's keys are 960..999
        k[:, :, j, :] = 0.0
        k[:, :, j, 0] = beta
    qs, ks, vs = _to16(q, dtype), _to16(k, dtype), _to16(v, dtype)
    O, L = oracle.attention(_f64(qs, dtype), _f64(ks, dtype), _f64(vs, dtype), scale)
    return qs, ks, vs, O, L


def _dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return dev_bf16(a)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _seq(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a.transpose(0, 2, 1, 3))


def assert_parity(o, lse, O, L, dtype, what):
    if dtype == "bf16":
        assert_bf16_parity(o, lse, O, L, what)
        return
    d = np.abs(o - O)
    rel = float(np.linalg.norm(o - O) / np.linalg.norm(O))
    lse_err = float(np.max(np.abs(lse - L)))
    log(f"  {what}: O max-abs {d.max():.3e} mean-abs {d.mean():.3e} rel-L2 {rel:.3e}; LSE max-abs {lse_err:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert rel <= F16_REL_L2, rel
    assert lse_err <= F16_LSE_MAX_ABS, lse_err


def test_planted_raise_fires():
    """(CPU) The planted scores do raise m by more than 2^8 over the first block's max (base 2) for
    nearly every row, and the keys before the planted one keep a visible share of the weight in
    the moderate case (CPU check of the construction)."""
    log("case: planted-raise construction")
    for kind in KIND_DELTA:
        qs, ks, _, _, _ = case_data(kind, "late", "bf16")
        q, k = _f64(qs, "bf16"), _f64(ks, "bf16")
        z = np.einsum("bhid,bhjd->bhij", q, k) * scale_of(D) / np.log(2.0)     # base-2 scores
        first = z[..., :64].max(axis=-1)
        planted = z[..., 14 * 64:15 * 64].max(axis=-1)
        frac = float(np.mean(planted > first + 8.0))
        before = np.exp(np.log(2.0) * (z[..., :14 * 64] - z.max(axis=-1, keepdims=True))).sum(-1)
        total = np.exp(np.log(2.0) * (z - z.max(axis=-1, keepdims=True))).sum(-1)
        share = float(np.median(before / total))
        log(f"  {kind}: raise at block 14 for {frac:.4f} of rows; weight of blocks 0-13 (median) {share:.3e}")
        assert frac >= 0.99
        if kind == "moderate":
            assert 0.02 <= share <= 0.5


@pytest.mark.gpu
@pytest.mark.parametrize("split", [False, True], ids=["unsplit", "split"])
@pytest.mark.parametrize("seq_major", [False, True], ids=["bhsd", "bshd"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("placement", list(PLACEMENT_BLOCK))
@pytest.mark.parametrize("kind", list(KIND_DELTA))
def test_planted_raise(kind, placement, dtype, seq_major, split):
    log(f"case: planted raise kind={kind} placement={placement} dtype={dtype} seq_major={seq_major} split={split}")
    qs, ks, vs, O, L = case_data(kind, placement, dtype)
    tr = _seq if seq_major else (lambda a: a)
    code = cp.BF16 if dtype == "bf16" else cp.F16
    ws = None
    if split:
        n = cp.attn_fwd_workspace_size(B, H, SQ, SKV, D, code, code)
        assert n > 0, "the planner was expected to split this shape"
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    q, k, v = (_dev(tr(a), dtype) for a in (qs, ks, vs))
    o, lse = cp.attn_fwd_ex(q, k, v, workspace=ws, seq_major=seq_major)
    torch.cuda.synchronize()
    og = host64(o.transpose(1, 2) if seq_major else o)
    assert_parity(og, host64(lse), O, L, dtype, f"{kind}/{placement}/{dtype}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kind", list(KIND_DELTA))
def test_planted_raise_f32_out(kind, dtype):
    """The same raise with an f32 O (the ring-partial format): no output rounding, so the error
    is the weight rounding alone."""
    log(f"case: planted raise f32 O kind={kind} dtype={dtype}")
    qs, ks, vs, O, L = case_data(kind, "late", dtype)
    o, lse = cp.attn_fwd(*(_dev(a, dtype) for a in (qs, ks, vs)), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(host64(o), host64(lse), O, L, dtype, f"{kind}/f32 O/{dtype}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_planted_raise_accumulate(dtype):
    """Ring-style accumulation over two key chunks where the raise happens inside the second
    chunk: chunk 1 folds into chunk 0's f32 (O, LSE) through the accumulate epilogue."""
    log(f"case: planted raise accumulated over two chunks dtype={dtype}")
    qs, ks, vs, O, L = case_data("moderate", "late", dtype)
    q = _dev(qs, dtype)
    o = torch.empty((B, H, SQ, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, SQ), dtype=torch.float32, device="cuda")
    cut = 512
    for c, (lo, hi) in enumerate(((0, cut), (cut, SKV))):
        k = _dev(np.ascontiguousarray(ks[:, :, lo:hi]), dtype)
        v = _dev(np.ascontiguousarray(vs[:, :, lo:hi]), dtype)
        cp.attn_fwd_ex(q, k, v, o=o, lse=lse, accumulate=c > 0)
    torch.cuda.synchronize()
    assert_parity(host64(o), host64(lse), O, L, dtype, f"moderate/accumulate/{dtype}")
