"""C-ABI checks that need no GPU.

The library must load, export every function include/cpattn.h declares, and
reject bad arguments with the documented status before any HIP call.  The
pointers passed here are fake addresses that are never dereferenced: every
call below fails validation, so nothing is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

from long_sequence_bidirectional_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")

A = 0x10000000      # fake, 16-byte aligned, far apart
B_ = 0x20000000
C = 0x30000000
D_ = 0x40000000
E = 0x50000000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libcpattn.so not built (run python -m long_sequence_bidirectional_amd.build)")
    return _lib.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpattn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert header_functions() == sorted(["cpattn_abi_version", "cpattn_attn_fwd", "cpattn_attn_fwd_ex",
                                         "cpattn_attn_fwd_ex_static", "cpattn_attn_fwd_fp8",
                                         "cpattn_attn_fwd_split_plan", "cpattn_attn_fwd_workspace_size",
                                         "cpattn_attn_merge", "cpattn_qk_rmsnorm", "cpattn_ring_attn_fwd",
                                         "cpattn_status_string",
                                         "cpattn_ulysses_pack", "cpattn_ulysses_pack_n",
                                         "cpattn_ulysses_unpack", "cpattn_ulysses_unpack_n"])


def test_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (cpattn_\w+)", out))
    assert set(header_functions()) <= exported
    # nothing else leaks out of the C ABI
    assert {s for s in exported if s.startswith("cpattn")} == set(header_functions())
    assert {name for name, _, _ in _lib.SIGNATURES} == set(header_functions())


def test_version_and_status_strings(L):
    assert L.cpattn_abi_version() == _lib.ABI_VERSION == 4
    seen = set()
    for s in range(10):
        msg = L.cpattn_status_string(s)
        assert msg and msg not in seen
        seen.add(msg)
    assert L.cpattn_status_string(99) == b"unknown status"


def fwd(L, q=A, k=B_, v=C, o=D_, lse=E, B=1, H=2, Sq=256, Skv=256, D=64, scale=0.125, i=0, od=0):
    return L.cpattn_attn_fwd(q, k, v, o, lse, B, H, Sq, Skv, D, scale, i, od, None)


def test_attn_fwd_validation(L):
    assert fwd(L, q=None) == _lib.E_NULL
    assert fwd(L, o=None) == _lib.E_NULL
    assert fwd(L, lse=None) == _lib.E_NULL
    assert fwd(L, k=None) == _lib.E_NULL
    assert fwd(L, i=2) == _lib.E_DTYPE
    assert fwd(L, i=_lib.F32, od=_lib.BF16) == _lib.E_DTYPE
    assert fwd(L, i=_lib.F16, od=_lib.BF16) == _lib.E_DTYPE           # O in the input type or f32
    assert fwd(L, i=_lib.BF16, od=_lib.F16) == _lib.E_DTYPE
    assert fwd(L, i=_lib.F32, od=_lib.F16) == _lib.E_DTYPE
    assert fwd(L, i=3) == _lib.E_DTYPE
    assert fwd(L, D=96) == _lib.E_HEADDIM
    assert fwd(L, D=256) == _lib.E_HEADDIM
    assert fwd(L, B=0) == _lib.E_SHAPE
    assert fwd(L, Sq=0) == _lib.E_SHAPE
    assert fwd(L, Skv=-1) == _lib.E_SHAPE
    assert fwd(L, H=1 << 31) == _lib.E_SHAPE
    assert fwd(L, B=1 << 30, H=1 << 30, Sq=1 << 30) == _lib.E_SHAPE   # element count overflow
    assert fwd(L, scale=0.0) == _lib.E_SCALE
    assert fwd(L, scale=-0.1) == _lib.E_SCALE
    assert fwd(L, scale=float("inf")) == _lib.E_SCALE
    assert fwd(L, scale=float("nan")) == _lib.E_SCALE
    assert fwd(L, q=A + 8) == _lib.E_ALIGN
    assert fwd(L, lse=E + 4) == _lib.E_ALIGN
    # o overlapping q, lse overlapping o, lse overlapping v
    assert fwd(L, o=A + 16) == _lib.E_ALIAS
    assert fwd(L, lse=D_ + 64) == _lib.E_ALIAS
    assert fwd(L, lse=C + 1024) == _lib.E_ALIAS


W = 0x60000000     # fake workspace


def fwd_ex(L, q=A, k=B_, v=C, o=D_, lse=E, B=1, H=2, Sq=256, Skv=256, D=64, scale=0.125, i=0, od=0, flags=0,
           ws=W, ws_bytes=1 << 20):
    return L.cpattn_attn_fwd_ex(q, k, v, o, lse, B, H, Sq, Skv, D, scale, i, od, flags, ws, ws_bytes, None)


def test_attn_fwd_ex_validation(L):
    # the attn_fwd checks apply unchanged
    assert fwd_ex(L, q=None) == _lib.E_NULL
    assert fwd_ex(L, i=_lib.F32, od=_lib.BF16) == _lib.E_DTYPE
    assert fwd_ex(L, D=96) == _lib.E_HEADDIM
    assert fwd_ex(L, scale=0.0) == _lib.E_SCALE
    assert fwd_ex(L, o=A + 16) == _lib.E_ALIAS
    # flags
    assert fwd_ex(L, flags=8) == _lib.E_FLAGS
    assert fwd_ex(L, flags=_lib.FLAG_SEQ_MAJOR | 8) == _lib.E_FLAGS
    assert fwd_ex(L, flags=0x80000000) == _lib.E_FLAGS
    # the layout flag keeps every other check
    assert fwd_ex(L, flags=_lib.FLAG_SEQ_MAJOR, q=None) == _lib.E_NULL
    assert fwd_ex(L, flags=_lib.FLAG_SEQ_MAJOR, o=A + 16) == _lib.E_ALIAS
    assert fwd_ex(L, flags=_lib.FLAG_SEQ_MAJOR | _lib.FLAG_ACCUMULATE, od=_lib.BF16) == _lib.E_DTYPE
    # a token row of H * D >= 2^25 elements does not fit the kernels' 32-bit block offsets
    # (one row of q/k/v/o: 64 MiB each, inside the fake buffers' 256 MiB spacing)
    assert fwd_ex(L, flags=_lib.FLAG_SEQ_MAJOR, H=1 << 19, Sq=1, Skv=1, ws=None, ws_bytes=0) == _lib.E_SHAPE
    # accumulate needs bf16 inputs and an f32 accumulator
    assert fwd_ex(L, flags=_lib.FLAG_ACCUMULATE, od=_lib.BF16) == _lib.E_DTYPE
    assert fwd_ex(L, flags=_lib.FLAG_ACCUMULATE, i=_lib.F32, od=_lib.F32) == _lib.E_DTYPE
    # workspace
    assert fwd_ex(L, ws=None) == _lib.E_NULL                 # NULL with a size
    assert fwd_ex(L, ws=W + 8) == _lib.E_ALIGN
    assert fwd_ex(L, ws=A + 4096) == _lib.E_ALIAS            # on top of q
    assert fwd_ex(L, ws=D_ - 4096, ws_bytes=8192) == _lib.E_ALIAS   # runs into o
    assert fwd_ex(L, ws=E, ws_bytes=16) == _lib.E_ALIAS      # on top of lse


def fwd_static(L, q=A, k=B_, v=C, o=D_, lse=E, B=1, H=2, Sq=256, Skv=256, D=64, scale=0.125, i=0, od=0, flags=0,
               nbytes=1 << 20):
    return L.cpattn_attn_fwd_ex_static(q, k, v, o, lse, B, H, Sq, Skv, D, scale, i, od, flags, nbytes, None)


def test_k_seq_last_validation(L):
    """CPATTN_FLAG_K_SEQ_LAST: 16-bit inputs only, not with the sequence-major layout, Skv a
    multiple of 8 and D * Skv * 2 below 2^32; the fp8 entry point does not take the flag."""
    KT = 4
    def ex(flags, i=0, od=0, Skv=256, D=64, q=A, k=B_, v=C, o=D_, lse=E):
        return L.cpattn_attn_fwd_ex(q, k, v, o, lse, 1, 2, 256, Skv, D, 0.125, i, od, flags, None, 0, None)
    assert ex(KT | 2) == _lib.E_FLAGS
    assert ex(KT, i=_lib.F32, od=_lib.F32) == _lib.E_DTYPE
    assert ex(KT, Skv=260) == _lib.E_SHAPE
    far = [(i + 1) << 44 for i in range(5)]
    assert ex(KT, Skv=1 << 24, D=128, q=far[0], k=far[1], v=far[2], o=far[3], lse=far[4]) == _lib.E_SHAPE
    assert ex(8) == _lib.E_FLAGS
    assert L.cpattn_attn_fwd_fp8(A, B_, C, D_, E, 1, 2, 256, 256, 128, 0.1, 1.0, 1.0, 1.0, 0, KT, None, 0,
                                 None) == _lib.E_FLAGS


def test_binding_k_seq_last_shapes():
    import torch
    import long_sequence_bidirectional_amd as cp
    q = torch.zeros((1, 2, 16, 64), dtype=torch.bfloat16)
    v = torch.zeros((1, 2, 24, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape mismatch"):
        cp.attn_fwd_ex(q, torch.zeros((1, 2, 24, 64), dtype=torch.bfloat16), v, k_seq_last=True)
    with pytest.raises(ValueError, match="head-major"):
        cp.attn_fwd_ex(q, torch.zeros((1, 2, 64, 24), dtype=torch.bfloat16), v, seq_major=True, k_seq_last=True)


def test_binding_accumulate_needs_outputs():
    """Accumulating folds into the (o, lse) already there, so every binding that accumulates
    refuses a call without them before it allocates or touches a device (the fp8 binding once
    allocated fresh outputs first, which made its check dead)."""
    import torch
    import long_sequence_bidirectional_amd as cp
    q = torch.zeros((1, 2, 16, 128), dtype=torch.bfloat16)
    kv = torch.zeros((1, 2, 24, 128), dtype=torch.bfloat16)
    q8, kv8 = q.to(torch.uint8), kv.to(torch.uint8)
    for fn, args in ((cp.attn_fwd_ex, (q, kv, kv)), (cp.attn_fwd_ex_static, (q, kv, kv)),
                     (cp.attn_fwd_fp8, (q8, kv8, kv8))):
        with pytest.raises(ValueError, match="accumulate needs"):
            fn(*args, accumulate=True)
        with pytest.raises(ValueError, match="accumulate needs"):
            fn(*args, lse=torch.zeros((1, 2, 16)), accumulate=True)


def test_attn_fwd_ex_static_validation(L):
    """Every check of attn_fwd_ex except the workspace pointer's, plus the scratch limit; all of
    them run before the one HIP call (the lookup of the scratch's device address)."""
    limit = 32 << 20
    assert _lib.STATIC_SCRATCH_BYTES == limit
    m = re.search(r"#define CPATTN_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == limit
    assert fwd_static(L, nbytes=limit + 1) == _lib.E_SHAPE
    assert fwd_static(L, nbytes=2 ** 64 - 1) == _lib.E_SHAPE
    assert fwd_static(L, q=None) == _lib.E_NULL
    assert fwd_static(L, i=_lib.F32, od=_lib.BF16) == _lib.E_DTYPE
    assert fwd_static(L, D=96) == _lib.E_HEADDIM
    assert fwd_static(L, scale=float("nan")) == _lib.E_SCALE
    assert fwd_static(L, o=A + 16) == _lib.E_ALIAS
    assert fwd_static(L, flags=8) == _lib.E_FLAGS
    assert fwd_static(L, flags=_lib.FLAG_ACCUMULATE, od=_lib.BF16) == _lib.E_DTYPE
    assert fwd_static(L, flags=_lib.FLAG_SEQ_MAJOR, H=1 << 19, Sq=1, Skv=1) == _lib.E_SHAPE


def plan(L, B=1, H=24, Sq=44160, Skv=44160, D=128, slots=256, ws=2**64 - 1):
    t, p, b = ctypes.c_int64(-1), ctypes.c_int64(-1), ctypes.c_uint64(1)
    st = L.cpattn_attn_fwd_split_plan(B, H, Sq, Skv, D, slots, ws, ctypes.byref(t), ctypes.byref(p),
                                      ctypes.byref(b))
    assert st == _lib.OK
    return t.value, p.value, b.value


def piece_bytes(D):
    return 256 * (D + 1) * 4


SCHED = 2048       # bytes of dynamic-schedule counters at the head of every workspace


def test_counter_area_constant():
    m = re.search(r"#define CPATTN_WORKSPACE_COUNTER_BYTES (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == SCHED == _lib.SCHED_BYTES


def test_split_plan(L):
    """The planner's choices, worked out by hand for 256 resident workgroups (one per CU):
    T tiles of 256 rows leave T mod 256 tiles for the last wave; s pieces of those cost
    ceil(rem*s/256) * (1/s + 4/nblk) tile-times against 1 for no split, with s <= nblk / 8.  Every workspace
    starts with SCHED bytes of schedule counters; the pieces take the rest."""
    # video self-attention: 24 * 173 = 4152 tiles, 56 in the last wave, 690 key blocks.
    # One round: s = 4 (56 * 4 <= 256) costs 0.2558; two rounds of s = 9 (504 pieces)
    # cost 2 * (1/9 + 4/690) = 0.2338, the minimum
    assert plan(L) == (56, 9, SCHED + 56 * 9 * piece_bytes(128))
    # AllGather-KV rank: 24 * 22 = 528 tiles, 16 left over -> 16 pieces each (0.0683)
    assert plan(L, Sq=5520) == (16, 16, SCHED + 256 * piece_bytes(128))
    # Ulysses rank: 3 * 173 = 519 tiles, 7 left over -> 36 pieces (252 <= 256; 0.0336)
    assert plan(L, H=3) == (7, 36, SCHED + 252 * piece_bytes(128))
    # ring chunk: 528 tiles against 87 key blocks: s <= 10 by the 8-block minimum; 10 (0.146)
    assert plan(L, Sq=5520, Skv=5520) == (16, 10, SCHED + 160 * piece_bytes(128))
    # a full last wave: nothing to split (the counters are still used)
    assert plan(L, H=16, Sq=4096) == (0, 1, SCHED)
    # 250 of 256 slots busy in the last wave: splitting cannot beat one round
    assert plan(L, H=22, Sq=5888) == (0, 1, SCHED)
    # fewer than 16 key blocks (two pieces of 8): never split
    assert plan(L, H=1, Sq=300, Skv=448) == (0, 1, SCHED)
    assert plan(L, H=1, Sq=300, Skv=960) == (0, 1, SCHED)
    assert plan(L, H=1, Sq=300, Skv=1024) == (2, 2, SCHED + 4 * piece_bytes(128))
    # few tiles, few keys: 8 tiles, 47 blocks -> at most 5 pieces of >= 8 blocks
    assert plan(L, H=2, Sq=1000, Skv=3000) == (8, 5, SCHED + 40 * piece_bytes(128))
    # the workspace bounds the pieces: room for 100 -> 6 per tile of 16
    assert plan(L, Sq=5520, ws=SCHED + 100 * piece_bytes(128) + 5) == (16, 6, SCHED + 96 * piece_bytes(128))
    # room for fewer than two pieces per tile, or no slots known: no split
    assert plan(L, Sq=5520, ws=SCHED + 31 * piece_bytes(128)) == (0, 1, SCHED)
    assert plan(L, slots=0) == (0, 1, SCHED)
    # less than the counter area: no workspace at all (static schedule, no split)
    assert plan(L, Sq=5520, ws=SCHED - 1) == (0, 1, 0)
    # D = 64 pieces are smaller
    assert plan(L, H=3, D=64) == (7, 36, SCHED + 252 * piece_bytes(64))


def test_split_plan_validation(L):
    t, p, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_uint64()
    f = L.cpattn_attn_fwd_split_plan
    assert f(1, 2, 100, 100, 128, 256, 0, None, ctypes.byref(p), ctypes.byref(b)) == _lib.E_NULL
    assert f(1, 2, 0, 100, 128, 256, 0, ctypes.byref(t), ctypes.byref(p), ctypes.byref(b)) == _lib.E_SHAPE
    assert f(1, 2, 100, 100, 96, 256, 0, ctypes.byref(t), ctypes.byref(p), ctypes.byref(b)) == _lib.E_HEADDIM
    assert f(1, 2, 100, 100, 128, -1, 0, ctypes.byref(t), ctypes.byref(p), ctypes.byref(b)) == _lib.E_SHAPE
    n = ctypes.c_uint64()
    assert L.cpattn_attn_fwd_workspace_size(1, 2, 100, 100, 128, 0, 0, None) == _lib.E_NULL
    assert L.cpattn_attn_fwd_workspace_size(1, 2, 100, 100, 128, 7, 0, ctypes.byref(n)) == _lib.E_DTYPE
    assert L.cpattn_attn_fwd_workspace_size(1, 2, 100, 100, 48, 0, 0, ctypes.byref(n)) == _lib.E_HEADDIM
    # E4M3 inputs: D = 128 and a BF16 or F32 O only
    assert L.cpattn_attn_fwd_workspace_size(1, 2, 100, 100, 64, _lib.E4M3, 0, ctypes.byref(n)) == _lib.E_HEADDIM
    assert L.cpattn_attn_fwd_workspace_size(1, 2, 100, 100, 128, _lib.E4M3, _lib.F16, ctypes.byref(n)) == \
        _lib.E_DTYPE
    assert L.cpattn_attn_fwd_workspace_size(1, 2, 100, 100, 128, 4, 0, ctypes.byref(n)) == _lib.E_DTYPE
    # f32 inputs never split: answered without asking the device
    assert L.cpattn_attn_fwd_workspace_size(1, 2, 100, 100, 128, 1, 1, ctypes.byref(n)) == _lib.OK
    assert n.value == 0


def merge(L, oa=A, la=B_, ob=C, lb=D_, oo=E, lo=0x60000000, B=1, H=2, S=100, D=128, dt=0):
    return L.cpattn_attn_merge(oa, la, ob, lb, oo, lo, B, H, S, D, dt, None)


def test_attn_merge_validation(L):
    assert merge(L, oa=None) == _lib.E_NULL
    assert merge(L, lo=None) == _lib.E_NULL
    assert merge(L, dt=5) == _lib.E_DTYPE
    assert merge(L, S=0) == _lib.E_SHAPE
    assert merge(L, D=4) == _lib.E_HEADDIM
    assert merge(L, D=12) == _lib.E_HEADDIM            # 24 bytes per row: not a multiple of 16
    assert merge(L, D=2048) == _lib.E_HEADDIM
    assert merge(L, oo=E + 2) == _lib.E_ALIGN
    assert merge(L, oo=A + 256) == _lib.E_ALIAS        # partial overlap with o_a
    assert merge(L, lo=B_ + 16) == _lib.E_ALIAS        # partial overlap with lse_a
    assert merge(L, oo=B_) == _lib.E_ALIAS             # o_out on top of lse_a


def test_attn_merge_launch_size_limit(L):
    """A merge launch holds fewer than 2^32 work-items; larger shapes are refused as E_SHAPE
    before any HIP call (only the refusing side is probed: these fake buffers must never reach a
    kernel).  Work-items per launch: 256 per workgroup; f32 D=128 rows take 2 rows per wave and
    4 waves per workgroup, bf16 D=8 rows 64 per wave, f32 D=1024 rows one wave each."""
    far = [(i + 1) << 40 for i in range(6)]              # 1 TiB apart: no overlap at these sizes
    lim_wg = (1 << 24) - 1                                 # workgroups of 256 below 2^32 work-items
    for D, dt, rows_per_wg in ((128, _lib.F32, 8), (8, _lib.BF16, 256), (1024, _lib.F32, 4)):
        rows = lim_wg * rows_per_wg + 2                    # one workgroup more than fits
        st = L.cpattn_attn_merge(*far, 1, 2, rows // 2, D, dt, None)
        assert st == _lib.E_SHAPE, (D, dt, st)


def test_relayout_row_index_limit(L):
    # more than 2^32 rows of D values do not fit the kernel's 32-bit row indices
    assert rl(L, "cpattn_ulysses_pack", src=1 << 40, dst=1 << 44, S_l=(1 << 31) - 1, H=8, P=8) == _lib.E_SHAPE
    # a row of 2^31 or more 16-byte chunks does not fit its 32-bit chunk index within a row
    assert rl(L, "cpattn_ulysses_pack", src=1 << 40, dst=1 << 46, B=1, S_l=1, H=8, P=8, D=1 << 34) == _lib.E_SHAPE


def test_binding_refuses_undivided_relayout():
    """The binding derives S_local = S // P for a head->seq pack: an S that P does not divide
    would be read with the wrong per-head stride, so it is refused before any device call (as
    the oracle refuses it); likewise a head count that P does not divide."""
    import torch
    import long_sequence_bidirectional_amd as cp
    with pytest.raises(ValueError, match="divisible"):
        cp.ulysses_pack(torch.zeros((1, 3, 100, 128), dtype=torch.bfloat16), 8, cp.HEAD_TO_SEQ)
    with pytest.raises(ValueError, match="divisible"):
        cp.ulysses_pack(torch.zeros((1, 10, 20, 128), dtype=torch.bfloat16), 8, cp.SEQ_TO_HEAD)
    import oracle
    with pytest.raises(ValueError):
        oracle.ulysses_pack(torch.zeros((1, 3, 100, 128)).numpy(), 8, oracle.HEAD_TO_SEQ)


def ring(L, q=A, k=B_, v=C, o=D_, lse=E, ow=0x60000000, lw=0x70000000, n=8, Skv=64, D=128, scale=0.1):
    return L.cpattn_ring_attn_fwd(q, k, v, o, lse, ow, lw, 1, 2, 64, Skv, n, D, scale, None)


def test_ring_validation(L):
    assert ring(L, q=None) == _lib.E_NULL
    assert ring(L, ow=None) == _lib.E_NULL             # one work buffer without the other
    assert ring(L, lw=None) == _lib.E_NULL
    assert ring(L, n=0) == _lib.E_SHAPE
    assert ring(L, D=80) == _lib.E_HEADDIM
    assert ring(L, scale=0.0) == _lib.E_SCALE
    assert ring(L, lw=E + 16) == _lib.E_ALIAS          # workspace LSE overlaps LSE
    assert ring(L, ow=B_ + 4096) == _lib.E_ALIAS       # workspace O overlaps the K chunks


def fp8(L, q=A, k=B_, v=C, o=D_, lse=E, B=1, H=2, Sq=256, Skv=256, D=128, scale=0.1, qs=1.0, ks=1.0, vs=1.0,
        od=0, flags=0, ws=None, ws_bytes=0):
    return L.cpattn_attn_fwd_fp8(q, k, v, o, lse, B, H, Sq, Skv, D, scale, qs, ks, vs, od, flags, ws, ws_bytes, None)


def test_attn_fwd_fp8_validation(L):
    assert fp8(L, q=None) == _lib.E_NULL
    assert fp8(L, k=None) == _lib.E_NULL
    assert fp8(L, od=_lib.F16) == _lib.E_DTYPE
    assert fp8(L, D=64) == _lib.E_HEADDIM
    assert fp8(L, D=96) == _lib.E_HEADDIM
    assert fp8(L, Sq=0) == _lib.E_SHAPE
    assert fp8(L, scale=0.0) == _lib.E_SCALE
    assert fp8(L, qs=0.0) == _lib.E_SCALE
    assert fp8(L, vs=float("inf")) == _lib.E_SCALE
    assert fp8(L, flags=4) == _lib.E_FLAGS
    assert fp8(L, flags=_lib.FLAG_ACCUMULATE | 8) == _lib.E_FLAGS
    assert fp8(L, flags=_lib.FLAG_ACCUMULATE, od=_lib.BF16) == _lib.E_DTYPE     # accumulate needs an f32 O
    # workspace checks as for attn_fwd_ex
    assert fp8(L, ws=None, ws_bytes=1024) == _lib.E_NULL
    assert fp8(L, ws=W + 8, ws_bytes=1024) == _lib.E_ALIGN
    assert fp8(L, ws=A + 4096, ws_bytes=1024) == _lib.E_ALIAS             # on top of q
    assert fp8(L, ws=E, ws_bytes=16) == _lib.E_ALIAS                       # on top of lse
    # a token row of H * D >= 2^25 bytes does not fit the kernel's 32-bit block offsets
    assert fp8(L, flags=_lib.FLAG_SEQ_MAJOR, H=1 << 18, Sq=1, Skv=1) == _lib.E_SHAPE
    assert fp8(L, o=E + 16) == _lib.E_ALIGN or fp8(L, o=E + 16) == _lib.E_ALIAS
    assert fp8(L, o=A + 1024) == _lib.E_ALIAS          # o on top of q
    assert fp8(L, lse=C + 64) == _lib.E_ALIAS          # lse on top of v


def qkn(L, x=A, w=B_, y=C, rows=100, D=128, eps=1e-6, s=0.3, dt=2):
    return L.cpattn_qk_rmsnorm(x, w, y, rows, D, eps, s, dt, None)


def test_qk_rmsnorm_validation(L):
    assert qkn(L, x=None) == _lib.E_NULL
    assert qkn(L, w=None) == _lib.E_NULL
    assert qkn(L, dt=_lib.F32) == _lib.E_DTYPE
    assert qkn(L, dt=7) == _lib.E_DTYPE
    for D in (4, 96, 1024):
        assert qkn(L, D=D) == _lib.E_HEADDIM
    assert qkn(L, rows=0) == _lib.E_SHAPE
    assert qkn(L, rows=1 << 40) == _lib.E_SHAPE
    assert qkn(L, eps=-1.0) == _lib.E_SCALE
    assert qkn(L, eps=float("nan")) == _lib.E_SCALE
    assert qkn(L, s=0.0) == _lib.E_SCALE
    assert qkn(L, s=float("inf")) == _lib.E_SCALE
    assert qkn(L, s=1e-30) == _lib.E_SCALE                # rounds to 0 in fp16
    assert qkn(L, s=1e6) == _lib.E_SCALE                  # overflows fp16
    assert qkn(L, y=C + 8) == _lib.E_ALIGN
    assert qkn(L, y=A + 256) == _lib.E_ALIAS              # partial overlap with x
    assert qkn(L, y=B_ - 16) == _lib.E_ALIAS              # runs into w


def rl(L, fn, src=A, dst=B_, B=1, S_l=5520, H=24, D=128, P=8, dt=0, d=0):
    return getattr(L, fn)(src, dst, B, S_l, H, D, P, dt, d, None)


@pytest.mark.parametrize("fn", ["cpattn_ulysses_pack", "cpattn_ulysses_unpack"])
def test_relayout_validation(L, fn):
    assert rl(L, fn, src=None) == _lib.E_NULL
    assert rl(L, fn, dt=3) == _lib.E_DTYPE
    assert rl(L, fn, H=20) == _lib.E_SHAPE             # H % P != 0
    assert rl(L, fn, P=0) == _lib.E_SHAPE
    assert rl(L, fn, d=2) == _lib.E_SHAPE
    assert rl(L, fn, D=4) == _lib.E_HEADDIM            # 8-byte rows
    assert rl(L, fn, dst=B_ + 8) == _lib.E_ALIGN
    assert rl(L, fn, dst=A + 1024) == _lib.E_ALIAS


def rln(L, fn, srcs, dsts, n=None, **kw):
    """Batched relayout with host arrays of fake device pointers (a None entry is a NULL one)."""
    sa = (ctypes.c_void_p * max(1, len(srcs)))(*srcs)
    da = (ctypes.c_void_p * max(1, len(dsts)))(*dsts)
    a = dict(B=1, S_l=5520, H=24, D=128, P=8, dt=0, d=0)
    a.update(kw)
    return getattr(L, fn)(sa, da, len(srcs) if n is None else n, a["B"], a["S_l"], a["H"], a["D"], a["P"],
                          a["dt"], a["d"], None)


@pytest.mark.parametrize("fn", ["cpattn_ulysses_pack_n", "cpattn_ulysses_unpack_n"])
def test_batched_relayout_validation(L, fn):
    """The batched relayout checks each tensor as the single call does, plus the count and the
    pairwise overlaps of every destination with every source and every other destination."""
    # one shard [1, 5520, 24, 128] bf16 is 33,914,880 bytes: 1 GiB apart never overlaps
    src = [(1 + i) << 30 for i in range(8)]
    dst = [(16 + i) << 30 for i in range(8)]
    gap = 33914880
    assert getattr(L, fn)(None, (ctypes.c_void_p * 1)(dst[0]), 1, 1, 5520, 24, 128, 8, 0, 0, None) == _lib.E_NULL
    assert getattr(L, fn)((ctypes.c_void_p * 1)(src[0]), None, 1, 1, 5520, 24, 128, 8, 0, 0, None) == _lib.E_NULL
    assert rln(L, fn, src[:3], dst[:3], n=0) == _lib.E_SHAPE
    assert rln(L, fn, src[:3], [dst[0], None, dst[2]]) == _lib.E_NULL
    assert rln(L, fn, [src[0], src[1], None], dst[:3]) == _lib.E_NULL
    assert rln(L, fn, src[:3], dst[:3], dt=3) == _lib.E_DTYPE
    assert rln(L, fn, src[:3], dst[:3], H=20) == _lib.E_SHAPE
    assert rln(L, fn, src[:3], dst[:3], D=4) == _lib.E_HEADDIM
    assert rln(L, fn, src[:3], [dst[0], dst[1] + 8, dst[2]]) == _lib.E_ALIGN
    assert rln(L, fn, src[:3], [dst[0], dst[1], src[0] + 1024]) == _lib.E_ALIAS      # dst 2 over src 0
    assert rln(L, fn, src[:3], [dst[0], dst[0] + gap - 16, dst[2]]) == _lib.E_ALIAS  # dst 1 over dst 0
    assert rln(L, fn, src[:3], dst[:3], S_l=(1 << 31) - 1) == _lib.E_SHAPE          # > 2^32 rows


def test_batched_relayout_count_limit(L):
    """More than CPATTN_MAX_RELAYOUT_TENSORS tensors is a shape error (before any pointer is read
    past the eighth)."""
    src = [(1 + i) << 30 for i in range(9)]
    dst = [(16 + i) << 30 for i in range(9)]
    assert rln(L, "cpattn_ulysses_pack_n", src, dst) == _lib.E_SHAPE


def test_binding_refuses_mixed_batched_relayout():
    import torch
    import long_sequence_bidirectional_amd as cp
    a = torch.zeros((1, 10, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="first one"):
        cp.ulysses_pack_n([a, torch.zeros((1, 11, 8, 128), dtype=torch.bfloat16)], 8, cp.SEQ_TO_HEAD)
    with pytest.raises(ValueError, match="1 to 8"):
        cp.ulysses_pack_n([a] * 9, 8, cp.SEQ_TO_HEAD)
    with pytest.raises(ValueError, match="1 to 8"):
        cp.ulysses_unpack_n([], 8, cp.SEQ_TO_HEAD)


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libcpattn.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()
