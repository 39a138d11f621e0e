"""A seeded sweep of random problem shapes and options against the oracle.

The hand-picked parity cases cover each option on its own; this sweep draws them
together at random (fixed seed, so the cases are the same on every run):

* 16-bit inputs (bf16 or fp16), D in {64, 128}, B in {1, 2}, H in 1..5, Sq in 1..800 and
  Skv in 0..1700 (empty key sets included), head-major, sequence-major or K stored
  sequence-last, 16-bit or f32 O, with or without a workspace (so with or without the
  key-range split and the dynamic schedule), and, for f32 O, optionally accumulating onto
  the result of a second key set -- bf16 gates against the oracle;
* f32 inputs (the f32 kernel), both layouts -- the 1e-5 gate;
* E4M3 inputs (the fp8 kernel), both layouts, both output types, optional workspace and
  accumulation -- the derived fp8 bound of tests/test_gpu_fp8.py.
"""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import assert_bf16_parity, assert_f32_parity, dev_bf16, f64_of_bf16, host64, log, scale_of
from test_gpu_fp8 import check_fp8, dev8

pytestmark = pytest.mark.gpu


def draw_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        layout = str(rng.choice(["head", "seq", "kt"]))
        Skv = int(rng.integers(0, 1700)) if rng.random() > 0.08 else 0
        if layout == "kt":
            Skv = max(8, Skv // 8 * 8)
        out_f32 = bool(rng.random() < 0.5)
        cases.append(dict(i=i, dt=str(rng.choice(["bf16", "f16"])), D=D, B=int(rng.integers(1, 3)),
                          H=int(rng.integers(1, 6)), Sq=int(rng.integers(1, 801)), Skv=Skv, layout=layout,
                          out_f32=out_f32, ws=bool(rng.random() < 0.6),
                          acc=out_f32 and bool(rng.random() < 0.6),
                          Skv2=int(rng.integers(1, 300))))
    return cases


CASES16 = draw_cases(36, 5150)


def _name(c):
    return (f"{c['i']}-{c['dt']}-D{c['D']}-B{c['B']}H{c['H']}-{c['Sq']}x{c['Skv']}-{c['layout']}"
            f"{'-o32' if c['out_f32'] else ''}{'-ws' if c['ws'] else ''}{'-acc' if c['acc'] else ''}")


def _inputs16(dt, shape, seed):
    if dt == "bf16":
        a = inputs.random_bf16(shape, seed)
        return a, f64_of_bf16(a)
    a = inputs.random_f16(shape, seed)
    return a, a.astype(np.float64)


def _dev16(dt, a):
    return dev_bf16(a) if dt == "bf16" else torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("c", CASES16, ids=_name)
def test_random_16bit(c):
    log(f"case: {_name(c)}")
    B, H, Sq, Skv, D, dt = c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dt"]
    seed = 5200 + 10 * c["i"]
    qa, q64 = _inputs16(dt, (B, H, Sq, D), seed)
    ka, k64 = _inputs16(dt, (B, H, Skv, D), seed + 1)
    va, v64 = _inputs16(dt, (B, H, Skv, D), seed + 2)
    seq = c["layout"] == "seq"
    tr = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))) if seq else (lambda a: a)
    q, v = _dev16(dt, tr(qa)), _dev16(dt, tr(va))
    k = _dev16(dt, np.ascontiguousarray(ka.transpose(0, 1, 3, 2)) if c["layout"] == "kt" else tr(ka))
    od = torch.float32 if c["out_f32"] else None
    ws = None
    if c["ws"]:
        n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D, cp.BF16 if dt == "bf16" else cp.F16,
                                       cp.F32 if c["out_f32"] else (cp.BF16 if dt == "bf16" else cp.F16))
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o = lse = None
    if c["acc"]:
        # fold onto the result of a second key set, computed by a plain call (K head-major there
        # when this call takes K sequence-last: the fold target does not depend on K's layout)
        k2a, k2 = _inputs16(dt, (B, H, c["Skv2"], D), seed + 3)
        v2a, v2 = _inputs16(dt, (B, H, c["Skv2"], D), seed + 4)
        o, lse = cp.attn_fwd_ex(q, _dev16(dt, tr(k2a)), _dev16(dt, tr(v2a)), out_dtype=torch.float32,
                                seq_major=seq)
        k64, v64 = np.concatenate([k2, k64], axis=2), np.concatenate([v2, v64], axis=2)
    o, lse = cp.attn_fwd_ex(q, k, v, o=o, lse=lse, out_dtype=od, workspace=ws, accumulate=c["acc"],
                            seq_major=seq, k_seq_last=c["layout"] == "kt")
    torch.cuda.synchronize()
    O, L = oracle.attention(q64, k64, v64, scale_of(D))
    og = host64(o.transpose(1, 2)) if seq else host64(o)
    if k64.shape[2] == 0:
        assert np.all(og == 0) and np.all(np.isneginf(host64(lse)))
        return
    assert_bf16_parity(og, host64(lse), O, L, _name(c))


CASES32 = [dict(i=i, D=D, B=B, H=H, Sq=Sq, Skv=Skv, seq=seq) for i, (D, B, H, Sq, Skv, seq) in enumerate([
    (64, 1, 2, 256, 256, False), (128, 2, 1, 33, 700, True), (64, 1, 3, 129, 1, False), (128, 1, 1, 500, 31, True),
    (64, 2, 2, 77, 95, True), (128, 1, 2, 300, 1024, False)])]


@pytest.mark.parametrize("c", CASES32, ids=lambda c: f"{c['i']}-D{c['D']}-B{c['B']}H{c['H']}-{c['Sq']}x{c['Skv']}"
                                                    f"{'-seq' if c['seq'] else ''}")
def test_random_f32(c):
    B, H, Sq, Skv, D, seq = c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["seq"]
    log(f"case: f32 B{B} H{H} Sq{Sq} Skv{Skv} D{D} seq_major={seq}")
    seed = 5600 + 10 * c["i"]
    q, k, v = (inputs.random_f32(s, seed + j) for j, s in enumerate([(B, H, Sq, D), (B, H, Skv, D), (B, H, Skv, D)]))
    tr = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))) if seq else (lambda a: a)
    dq, dk, dv = (torch.from_numpy(tr(a)).cuda() for a in (q, k, v))
    o, lse = cp.attn_fwd_ex(dq, dk, dv, seq_major=seq)
    torch.cuda.synchronize()
    O, L = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale_of(D))
    og = host64(o.transpose(1, 2)) if seq else host64(o)
    assert_f32_parity(og, host64(lse), O, L, f"f32 {c}")


CASES8 = [dict(i=i, B=B, H=H, Sq=Sq, Skv=Skv, seq=seq, out_f32=o32, ws=ws, acc=acc)
          for i, (B, H, Sq, Skv, seq, o32, ws, acc) in enumerate([
              (1, 2, 1, 1, False, False, False, False), (2, 3, 700, 1030, True, True, True, True),
              (1, 1, 257, 1664, False, True, True, False), (1, 4, 129, 63, True, False, True, False),
              (2, 2, 511, 2048, False, True, False, True), (1, 5, 64, 640, True, False, True, False)])]


@pytest.mark.parametrize("c", CASES8, ids=lambda c: f"{c['i']}-B{c['B']}H{c['H']}-{c['Sq']}x{c['Skv']}"
                                                   f"{'-seq' if c['seq'] else ''}{'-o32' if c['out_f32'] else ''}"
                                                   f"{'-ws' if c['ws'] else ''}{'-acc' if c['acc'] else ''}")
def test_random_fp8(c):
    B, H, Sq, Skv, D, seq = c["B"], c["H"], c["Sq"], c["Skv"], 128, c["seq"]
    log(f"case: fp8 {c}")
    seed = 5800 + 10 * c["i"]
    q8, k8, v8 = (inputs.random_e4m3(s, seed + j) for j, s in enumerate([(B, H, Sq, D), (B, H, Skv, D),
                                                                          (B, H, Skv, D)]))
    qs, ks, vs = 0.75, 1.25, 0.5
    tr = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))) if seq else (lambda a: a)
    od = torch.float32 if c["out_f32"] else None
    ws = None
    if c["ws"]:
        n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D, cp.E4M3, cp.F32 if c["out_f32"] else cp.BF16)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o = lse = None
    if c["acc"]:
        # start from an empty result (O = 0, LSE = -inf), the merge identity
        o = torch.zeros((B, Sq, H, D) if seq else (B, H, Sq, D), dtype=torch.float32, device="cuda")
        lse = torch.full((B, H, Sq), float("-inf"), dtype=torch.float32, device="cuda")
    o, lse = cp.attn_fwd_fp8(dev8(tr(q8)), dev8(tr(k8)), dev8(tr(v8)), qs, ks, vs, o=o, lse=lse, out_dtype=od,
                             seq_major=seq, workspace=ws, accumulate=c["acc"])
    torch.cuda.synchronize()
    og = o.transpose(1, 2) if seq else o
    check_fp8(q8, k8, v8, qs, ks, vs, scale_of(D), og, lse, f"fp8 {c}", out_f32=c["out_f32"])
