"""GPU parity at every small key-block count and around each 64-key block edge.

The attention kernels stream K/V in 64-key blocks through four LDS buffers: a
prologue loads the first three K blocks and two V blocks, each MFMA slot issues
the loads three blocks ahead, a remainder runs the last one to three blocks of
the unrolled loop, and a final slot does the last PV product alone.  Key counts
1..6 blocks (and one key either side of each block edge) exercise every such
path, in the bf16, fp16 and fp8 kernels, with and without a ragged query tile;
the split path is checked with pieces of four to five blocks, and key counts of
7..13 blocks cover the entry into and exit from the check-free steady-state
loop.  Oracle: exact fp64 attention of the same inputs; bounds as in the other
parity tests.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import assert_bf16_parity, dev_bf16, f64_of_bf16, host64, log, scale_of
from test_gpu_fp8 import check_fp8, dev8
from test_gpu_p4 import assert_f16_parity

pytestmark = pytest.mark.gpu

KEYS = [1, 2, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 319, 320, 321, 383, 384]


@pytest.mark.parametrize("Skv", KEYS)
@pytest.mark.parametrize("D", [128, 64])
def test_bf16_block_counts(Skv, D):
    B, H, Sq = 1, 2, 300
    log(f"case: bf16 B{B} H{H} Sq{Sq} Skv{Skv} D{D}")
    seed = 8000 + Skv + D
    qb = inputs.random_bf16((B, H, Sq, D), seed)
    kb = inputs.random_bf16((B, H, Skv, D), seed + 1)
    vb = inputs.random_bf16((B, H, Skv, D), seed + 2)
    o, lse = cp.attn_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb))
    torch.cuda.synchronize()
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(o), host64(lse), O, L, f"bf16 Skv={Skv} D={D}")


@pytest.mark.parametrize("Skv", KEYS)
def test_f16_block_counts(Skv):
    B, H, Sq, D = 1, 2, 300, 128
    log(f"case: fp16 B{B} H{H} Sq{Sq} Skv{Skv} D{D}")
    seed = 8100 + Skv
    q = inputs.random_f16((B, H, Sq, D), seed)
    k = inputs.random_f16((B, H, Skv, D), seed + 1)
    v = inputs.random_f16((B, H, Skv, D), seed + 2)
    o, lse = cp.attn_fwd(*(torch.from_numpy(x).cuda() for x in (q, k, v)))
    torch.cuda.synchronize()
    O, L = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale_of(D))
    assert_f16_parity(host64(o), host64(lse), O, L, f"fp16 Skv={Skv}")


@pytest.mark.parametrize("Skv", KEYS)
def test_fp8_block_counts(Skv):
    B, H, Sq, D = 1, 2, 300, 128
    log(f"case: fp8 B{B} H{H} Sq{Sq} Skv{Skv} D{D}")
    seed = 8200 + Skv
    q8 = inputs.random_e4m3((B, H, Sq, D), seed)
    k8 = inputs.random_e4m3((B, H, Skv, D), seed + 1)
    v8 = inputs.random_e4m3((B, H, Skv, D), seed + 2)
    o, lse = cp.attn_fwd_fp8(dev8(q8), dev8(k8), dev8(v8))
    torch.cuda.synchronize()
    check_fp8(q8, k8, v8, 1.0, 1.0, 1.0, 1.0 / math.sqrt(D), o, lse, f"fp8 Skv={Skv}")


@pytest.mark.parametrize("Skv", [1025, 1089, 1152, 1216, 1280])
def test_split_short_pieces(Skv):
    """Few tiles (all in the device's last, partial wave) and 17-20 key blocks: the planner cuts
    each tile into two pieces of eight to ten blocks, the shortest it makes."""
    B, H, Sq, D = 1, 2, 300, 128
    seed = 8300 + Skv
    qb = inputs.random_bf16((B, H, Sq, D), seed)
    kb = inputs.random_bf16((B, H, Skv, D), seed + 1)
    vb = inputs.random_bf16((B, H, Skv, D), seed + 2)
    n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D)
    tiles, pieces, _ = cp.attn_fwd_split_plan(B, H, Sq, Skv, D, 256, n)
    log(f"case: split B{B} H{H} Sq{Sq} Skv{Skv} D{D}: workspace {n} B, {tiles} tiles x {pieces} pieces")
    assert tiles > 0 and pieces >= 2
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    o, lse = cp.attn_fwd_ex(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), workspace=ws)
    torch.cuda.synchronize()
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(o), host64(lse), O, L, f"split Skv={Skv}")


# Key counts around the start of the check-free steady-state loop: it runs while every load of
# its four blocks is a full block (full blocks >= j + 7 for j = 1, 5, ...), then the checked
# loop, the remainder and the final slot take over; 7..13 blocks, full or with a ragged tail.
STEADY = [448, 449, 511, 512, 513, 575, 576, 577, 640, 641, 703, 704, 705, 767, 768, 769, 831, 832, 833]


@pytest.mark.parametrize("Skv", STEADY)
def test_bf16_steady_state_entry(Skv):
    B, H, Sq, D = 1, 2, 300, 128
    log(f"case: bf16 steady-state entry B{B} H{H} Sq{Sq} Skv{Skv} D{D}")
    seed = 8400 + Skv
    qb = inputs.random_bf16((B, H, Sq, D), seed)
    kb = inputs.random_bf16((B, H, Skv, D), seed + 1)
    vb = inputs.random_bf16((B, H, Skv, D), seed + 2)
    o, lse = cp.attn_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb))
    torch.cuda.synchronize()
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(o), host64(lse), O, L, f"bf16 Skv={Skv}")


@pytest.mark.parametrize("Skv", STEADY[::2])
def test_fp8_steady_state_entry(Skv):
    B, H, Sq, D = 1, 2, 300, 128
    log(f"case: fp8 steady-state entry B{B} H{H} Sq{Sq} Skv{Skv} D{D}")
    seed = 8500 + Skv
    q8 = inputs.random_e4m3((B, H, Sq, D), seed)
    k8 = inputs.random_e4m3((B, H, Skv, D), seed + 1)
    v8 = inputs.random_e4m3((B, H, Skv, D), seed + 2)
    o, lse = cp.attn_fwd_fp8(dev8(q8), dev8(k8), dev8(v8))
    torch.cuda.synchronize()
    check_fp8(q8, k8, v8, 1.0, 1.0, 1.0, 1.0 / math.sqrt(D), o, lse, f"fp8 Skv={Skv}")
