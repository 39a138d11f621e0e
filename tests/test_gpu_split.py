"""GPU parity of attn_fwd_ex: key-range split of the last wave, and accumulation.

The split cuts the keys of the query tiles in a partial last wave into pieces
and folds them with the merge rule; accumulation folds a call's result into an
existing (O, LSE).  Both are checked against the fp64 oracle on the whole
output, and against attn_fwd where the arithmetic is the same (bit-identical).
"""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import _lib, inputs
from helpers import assert_bf16_parity, dev_bf16, f64_of_bf16, host64, log, scale_of

pytestmark = pytest.mark.gpu


def workspace(B, H, Sq, Skv, D, out_f32=False):
    n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D, o_dtype=1 if out_f32 else 0)
    return torch.empty(n, dtype=torch.uint8, device="cuda"), n


def rand_qkv(B, H, Sq, Skv, D, seed):
    return (inputs.random_bf16((B, H, Sq, D), seed), inputs.random_bf16((B, H, Skv, D), seed + 1),
            inputs.random_bf16((B, H, Skv, D), seed + 2))


def same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


SPLIT_SHAPES = [
    (1, 2, 1000, 3000, 128),   # 8 tiles (ragged last), 47 key blocks (56-key tail): 5 pieces per tile
    (2, 3, 513, 1100, 64),     # D = 64, 18 tiles, 18 blocks (12-key tail): 2 pieces
    (1, 1, 17, 2992, 128),     # one tile of 17 rows, the text-token count (48-key tail)
    (1, 3, 300, 1080, 128),    # 17 blocks, 56-key tail: 2 pieces of 8 and 9 blocks
]


@pytest.mark.parametrize("out_f32", [False, True], ids=["o_bf16", "o_f32"])
@pytest.mark.parametrize("B,H,Sq,Skv,D", SPLIT_SHAPES)
def test_split_full(B, H, Sq, Skv, D, out_f32):
    log(f"case: split B{B} H{H} Sq{Sq} Skv{Skv} D{D} out_f32={out_f32}")
    qb, kb, vb = rand_qkv(B, H, Sq, Skv, D, 3000 + Sq + Skv + D)
    ws, n = workspace(B, H, Sq, Skv, D, out_f32)
    tiles, pieces, _ = cp.attn_fwd_split_plan(B, H, Sq, Skv, D, 256, n)
    log(f"  plan for 256 slots: {tiles} tiles x {pieces} pieces")
    assert n > _lib.SCHED_BYTES, "the planner was expected to split this shape"
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    od = torch.float32 if out_f32 else None
    o, lse = cp.attn_fwd_ex(q, k, v, out_dtype=od, workspace=ws)
    o_ref, lse_ref = cp.attn_fwd(q, k, v, out_dtype=od)
    torch.cuda.synchronize()
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(o), host64(lse), O, L, "split")
    d = torch.max(torch.abs(o.float() - o_ref.float())).item()
    log(f"  split vs unsplit: O max-abs {d:.3e}")
    assert d <= 2e-2


def test_workspace_size_bounds_the_split():
    B, H, Sq, Skv, D = 1, 2, 1000, 3000, 128
    qb, kb, vb = rand_qkv(B, H, Sq, Skv, D, 3100)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o_ref, l_ref = cp.attn_fwd(q, k, v)
    piece = 256 * (D + 1) * 4
    sched = _lib.SCHED_BYTES   # schedule counters at the head of the workspace
    # no workspace, or room for under two pieces per tile: the unsplit kernel, bit for bit
    # (the dynamic schedule with a workspace runs the same units with the same arithmetic)
    for nbytes in (0, sched - 1, sched + 3 * piece, sched + 15 * piece + 100):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o, l = cp.attn_fwd_ex(q, k, v, workspace=ws)
        torch.cuda.synchronize()
        log(f"  workspace {nbytes} B: unsplit")
        assert same_bits(o, o_ref) and same_bits(l, l_ref)
    # room for 2 or 5 pieces per tile: split, and still correct
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    for pieces in (2, 5):
        ws = torch.empty(sched + 8 * pieces * piece, dtype=torch.uint8, device="cuda")
        o, l = cp.attn_fwd_ex(q, k, v, workspace=ws)
        torch.cuda.synchronize()
        assert_bf16_parity(host64(o), host64(l), O, L, f"{pieces} pieces per tile")
        assert not same_bits(o, o_ref)


@pytest.mark.parametrize("B,H,Sq,Skv,D", [(1, 24, 4096, 256, 128),   # 384 tiles, 4 key blocks: no split
                                          (2, 12, 2600, 300, 64),    # 528 tiles (ragged), D = 64
                                          (1, 8, 44160, 200, 128)])  # 1384 tiles, 5 per slot
def test_dynamic_schedule_same_bits(B, H, Sq, Skv, D):
    """More tiles than resident workgroups and no split: with a workspace the units after the
    first round are claimed from a counter (dynamic schedule), without one they follow the static
    map; every unit runs the same arithmetic either way, so the results are the same bits.  The
    same workspace serves two calls in a row (the launcher clears its counters each time)."""
    log(f"case: dynamic schedule B{B} H{H} Sq{Sq} Skv{Skv} D{D}")
    qb, kb, vb = rand_qkv(B, H, Sq, Skv, D, 3150 + Sq)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    ws, n = workspace(B, H, Sq, Skv, D)
    assert n == _lib.SCHED_BYTES, "expected the counters only (no split)"
    o_ref, l_ref = cp.attn_fwd(q, k, v)
    for rep in range(2):
        # outputs start as NaN, so a unit that no workgroup ran would show
        o = torch.full_like(o_ref, float("nan"))
        l = torch.full_like(l_ref, float("nan"))
        cp.attn_fwd_ex(q, k, v, o=o, lse=l, workspace=ws)
        torch.cuda.synchronize()
        assert same_bits(o, o_ref) and same_bits(l, l_ref), f"call {rep}"


def test_whole_tiles_unchanged_by_split():
    """264 tiles on 256 slots: tiles 0..255 run whole and match attn_fwd bit for bit; the 8
    split tiles (head 23, rows 768..2815) match the oracle."""
    B, H, Sq, Skv, D = 1, 24, 2816, 1000, 128
    qb, kb, vb = rand_qkv(B, H, Sq, Skv, D, 3200)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    ws, n = workspace(B, H, Sq, Skv, D)
    log(f"case: 264 tiles, workspace {n} B")
    assert n > 0
    o, l = cp.attn_fwd_ex(q, k, v, workspace=ws)
    o_ref, l_ref = cp.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    # tiles below 21 * 11 = 231 are whole for any slot count >= 231 (MI355X: 256)
    assert same_bits(o[:, :21], o_ref[:, :21]) and same_bits(l[:, :21], l_ref[:, :21])
    O, L = oracle.attention(f64_of_bf16(qb[:, 21:]), f64_of_bf16(kb[:, 21:]), f64_of_bf16(vb[:, 21:]),
                            scale_of(D))
    assert_bf16_parity(host64(o[:, 21:]), host64(l[:, 21:]), O, L, "heads 21-23")


@pytest.mark.parametrize("use_ws", [False, True], ids=["no_ws", "ws"])
def test_accumulate_chunks_equals_unchunked(use_ws):
    D, H, Sq = 128, 2, 600
    edges = [0, 1000, 1001, 2600, 2650]
    qb, kb, vb = rand_qkv(1, H, Sq, edges[-1], D, 3300)
    q = dev_bf16(qb)
    o = torch.empty((1, H, Sq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H, Sq), dtype=torch.float32, device="cuda")
    for i, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
        k = dev_bf16(np.ascontiguousarray(kb[:, :, a:b]))
        v = dev_bf16(np.ascontiguousarray(vb[:, :, a:b]))
        ws = workspace(1, H, Sq, b - a, D, True)[0] if use_ws else None
        cp.attn_fwd_ex(q, k, v, o=o, lse=lse, workspace=ws, accumulate=i > 0)
    torch.cuda.synchronize()
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(o), host64(lse), O, L, f"4 chunks accumulated (workspace {use_ws})")


@pytest.mark.parametrize("use_ws", [False, True], ids=["no_ws", "ws"])
def test_accumulate_onto_empty_is_plain(use_ws):
    """Folding into the empty result (O = 0, LSE = -inf) is exact: weights 0 and 1."""
    B, H, Sq, Skv, D = 1, 2, 1000, 3000, 128
    qb, kb, vb = rand_qkv(B, H, Sq, Skv, D, 3400)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    ws = workspace(B, H, Sq, Skv, D, True)[0] if use_ws else None
    o_ref, l_ref = cp.attn_fwd_ex(q, k, v, out_dtype=torch.float32, workspace=ws)
    o = torch.zeros((B, H, Sq, D), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, Sq), float("-inf"), device="cuda")
    cp.attn_fwd_ex(q, k, v, o=o, lse=lse, workspace=ws, accumulate=True)
    torch.cuda.synchronize()
    assert same_bits(o, o_ref) and same_bits(lse, l_ref)


def test_accumulate_empty_keys_is_noop():
    D = 64
    q = dev_bf16(inputs.random_bf16((1, 2, 40, D), 3500))
    kv = torch.empty((1, 2, 0, D), dtype=torch.bfloat16, device="cuda")
    o = torch.randn((1, 2, 40, D), device="cuda")
    lse = torch.randn((1, 2, 40), device="cuda")
    o0, l0 = o.clone(), lse.clone()
    cp.attn_fwd_ex(q, kv, kv, o=o, lse=lse, accumulate=True)
    torch.cuda.synchronize()
    assert same_bits(o, o0) and same_bits(lse, l0)


@pytest.mark.parametrize("use_work", [False, True], ids=["no_work", "work"])
def test_ring_driver_with_split_chunks(use_work):
    n, Skv_c, Sq, D, H = 3, 1000, 600, 128, 2
    log(f"case: ring n{n} Skv_c{Skv_c} Sq{Sq} use_work={use_work}")
    qb = inputs.random_bf16((1, H, Sq, D), 3600)
    kcb = inputs.random_bf16((n, 1, H, Skv_c, D), 3601)
    vcb = inputs.random_bf16((n, 1, H, Skv_c, D), 3602)
    o, l = cp.ring_attn_fwd(dev_bf16(qb), dev_bf16(kcb), dev_bf16(vcb), use_work=use_work)
    torch.cuda.synchronize()
    k_all = np.concatenate([kcb[c] for c in range(n)], axis=2)
    v_all = np.concatenate([vcb[c] for c in range(n)], axis=2)
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(k_all), f64_of_bf16(v_all), scale_of(D))
    assert_bf16_parity(host64(o), host64(l), O, L, "ring with split chunks")


@pytest.mark.parametrize("H,Sq", [(2, 2304),       # 18 units per chunk: the shared counter only
                                  (8, 8448)])      # 264 units: per-XCD ranges of 32 and a tail of 8
def test_ring_driver_many_chunks(H, Sq):
    """35 chunks: chunk c takes schedule counter set c % 16 of the work buffers, and the sets are
    cleared once per 16 chunks (before chunks 0, 16 and 32), so later chunks reuse cleared sets."""
    n, Skv_c, D = 35, 130, 64                      # 3 key blocks per chunk (no split)
    log(f"case: ring n{n} Skv_c{Skv_c} H{H} Sq{Sq} D{D}")
    qb = inputs.random_bf16((1, H, Sq, D), 3700)
    kcb = inputs.random_bf16((n, 1, H, Skv_c, D), 3701)
    vcb = inputs.random_bf16((n, 1, H, Skv_c, D), 3702)
    q, kc, vc = dev_bf16(qb), dev_bf16(kcb), dev_bf16(vcb)
    o, l = cp.ring_attn_fwd(q, kc, vc)
    o2, l2 = cp.ring_attn_fwd(q, kc, vc, use_work=False)      # static schedule, same units
    torch.cuda.synchronize()
    assert same_bits(o, o2) and same_bits(l, l2)
    k_all = np.concatenate([kcb[c] for c in range(n)], axis=2)
    v_all = np.concatenate([vcb[c] for c in range(n)], axis=2)
    rows = np.array([0, 1, 255, 256, 1000, 2303, Sq - 1])
    O, L = oracle.attention_rows(f64_of_bf16(qb), f64_of_bf16(k_all), f64_of_bf16(v_all), scale_of(D), rows)
    assert_bf16_parity(host64(o[:, :, rows]), host64(l[:, :, rows]), O, L, "ring over 35 chunks")


@pytest.mark.parametrize("s", [3, 7, 20, 48])
def test_piece_merge_paths(s):
    """The piece merge reads a tile's pieces in one batch for up to 36 pieces (instantiated for
    4, 8, 12, 16, 24 and 36) and in batches beyond; the bench shapes use 4, 9, 10, 16 and 36
    pieces.  Here 258 tiles of one head on 256 slots leave 2 split tiles, 384 key blocks allow up
    to 48 pieces each, and the workspace size holds the plan to s pieces: 3, 7 and 20 take the
    4-, 8- and 24-piece forms, 48 the batched path.  Both output types; the f32 call accumulates
    onto the result of a separate key set, so the merge also folds in an existing row.  The split
    tiles' rows and a sample of whole-tile rows are checked against the oracle."""
    B, H, Sq, Skv, D = 1, 1, 258 * 256, 384 * 64, 128
    piece = 256 * (D + 1) * 4
    nbytes = _lib.SCHED_BYTES + 2 * s * piece
    tiles, pieces, used = cp.attn_fwd_split_plan(B, H, Sq, Skv, D, 256, nbytes)
    log(f"case: piece merge, {tiles} split tiles x {pieces} pieces (workspace {nbytes} B)")
    assert (tiles, pieces) == (2, s)
    qb, kb, vb = rand_qkv(B, H, Sq, Skv, D, 3400 + s)
    ka, va = inputs.random_bf16((B, H, 512, D), 3460 + s), inputs.random_bf16((B, H, 512, D), 3470 + s)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o16, l16 = cp.attn_fwd_ex(q, k, v, workspace=ws)
    o32, l32 = cp.attn_fwd(q, dev_bf16(ka), dev_bf16(va), out_dtype=torch.float32)
    cp.attn_fwd_ex(q, k, v, o=o32, lse=l32, workspace=ws, accumulate=True)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(256 * 256, Sq), inputs.sample_rows(256 * 256, 32, seed=3480 + s)])
    q64, k64, v64 = f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb)
    O, L = oracle.attention_rows(q64, k64, v64, scale_of(D), rows)
    assert_bf16_parity(host64(o16[:, :, rows]), host64(l16[:, :, rows]), O, L, f"{s} pieces, bf16 O")
    kc = np.concatenate([f64_of_bf16(ka), k64], axis=2)
    vc = np.concatenate([f64_of_bf16(va), v64], axis=2)
    O, L = oracle.attention_rows(q64, kc, vc, scale_of(D), rows)
    assert_bf16_parity(host64(o32[:, :, rows]), host64(l32[:, :, rows]), O, L, f"{s} pieces, f32 O accumulated")
