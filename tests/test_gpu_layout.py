"""GPU parity of sequence-major attention and of the fused DeepSpeed Ulysses path.

Sequence-major attention reads q [B,Sq,H,D] and k/v [B,Skv,H,D] and writes o
[B,Sq,H,D].  It must give bit for bit what the head-major call gives on the
transposed tensors, and match the oracle.  The fused Ulysses path (token
shards -> pack -> all-to-all -> attention on the receive buffer in place -> O
written into the send buffer -> all-to-all -> unpack) must equal attention
over the full sequence.  Ranks and the all-to-alls are simulated on one GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import (assert_bf16_parity, assert_f32_parity, dev_bf16, dev_f32, f64_of_bf16, host64, log,
                     scale_of)

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    v = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.contiguous().view(v), b.contiguous().view(v))


def seq(t):
    """[B,H,S,D] -> contiguous [B,S,H,D]."""
    return t.transpose(1, 2).contiguous()


SHAPES = [
    (1, 3, 300, 333, 128),    # ragged Q and KV tails, several tiles and blocks
    (2, 2, 513, 700, 64),     # batch 2, D = 64
    (1, 4, 17, 2992, 128),    # the text-token count
    (1, 1, 256, 64, 128),     # H = 1: both layouts are the same memory
]


@pytest.mark.parametrize("out_f32", [False, True], ids=["o_bf16", "o_f32"])
@pytest.mark.parametrize("B,H,Sq,Skv,D", SHAPES)
def test_seq_major_equals_head_major(B, H, Sq, Skv, D, out_f32):
    log(f"case: seq-major B{B} H{H} Sq{Sq} Skv{Skv} D{D} out_f32={out_f32}")
    seed = 4000 + Sq + Skv + D
    qb = inputs.random_bf16((B, H, Sq, D), seed)
    kb = inputs.random_bf16((B, H, Skv, D), seed + 1)
    vb = inputs.random_bf16((B, H, Skv, D), seed + 2)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    od = torch.float32 if out_f32 else None
    o_h, l_h = cp.attn_fwd(q, k, v, out_dtype=od)
    o_s, l_s = cp.attn_fwd_ex(seq(q), seq(k), seq(v), out_dtype=od, seq_major=True)
    torch.cuda.synchronize()
    assert same_bits(seq(o_h), o_s) and same_bits(l_h, l_s)
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(o_s.transpose(1, 2)), host64(l_s), O, L, "seq-major")


def test_seq_major_f32_inputs():
    B, H, Sq, Skv, D = 1, 3, 77, 130, 64
    q = inputs.random_f32((B, H, Sq, D), 4100)
    k = inputs.random_f32((B, H, Skv, D), 4101)
    v = inputs.random_f32((B, H, Skv, D), 4102)
    o, lse = cp.attn_fwd_ex(seq(dev_f32(q)), seq(dev_f32(k)), seq(dev_f32(v)), seq_major=True)
    torch.cuda.synchronize()
    O, L = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale_of(D))
    assert_f32_parity(host64(o.transpose(1, 2)), host64(lse), O, L, "f32 seq-major")


def test_seq_major_split_and_accumulate():
    """Key-range split and accumulation in the sequence-major layout: chunks of keys folded
    into one f32 accumulator equal the head-major fold bit for bit, and the oracle."""
    B, H, Sq, D = 1, 2, 1000, 128
    edges = [0, 1500, 1501, 3000]
    qb = inputs.random_bf16((B, H, Sq, D), 4200)
    kb = inputs.random_bf16((B, H, edges[-1], D), 4201)
    vb = inputs.random_bf16((B, H, edges[-1], D), 4202)
    q = dev_bf16(qb)
    outs = {}
    for seq_major in (False, True):
        o = torch.empty((B, Sq, H, D) if seq_major else (B, H, Sq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, Sq), device="cuda")
        for i, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
            k = dev_bf16(np.ascontiguousarray(kb[:, :, a:b]))
            v = dev_bf16(np.ascontiguousarray(vb[:, :, a:b]))
            n = cp.attn_fwd_workspace_size(B, H, Sq, b - a, D, o_dtype=1)
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
            if seq_major:
                cp.attn_fwd_ex(seq(q), seq(k), seq(v), o=o, lse=lse, workspace=ws, accumulate=i > 0, seq_major=True)
            else:
                cp.attn_fwd_ex(q, k, v, o=o, lse=lse, workspace=ws, accumulate=i > 0)
        outs[seq_major] = (o, lse)
    torch.cuda.synchronize()
    assert same_bits(seq(outs[False][0]), outs[True][0]) and same_bits(outs[False][1], outs[True][1])
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(outs[True][0].transpose(1, 2)), host64(outs[True][1]), O, L, "seq-major folded")


def alltoall(send):
    """Simulated all-to-all: send[r] is rank r's [B, P, S_l, Hp, D] buffer; rank r receives
    chunk r of every rank's buffer, chunk g coming from rank g."""
    P = len(send)
    return [torch.stack([send[g][:, r] for g in range(P)], dim=1).contiguous() for r in range(P)]


def ulysses_fused(shards_q, shards_k, shards_v, P, use_ws=False):
    """The per-rank Ulysses path with attention on the receive buffers in place.
    shards_*[r]: rank r's token shard [B, S_l, H, D].  Returns each rank's O shard [B, S_l, H, D]."""
    recv = {}
    for name, shards in (("q", shards_q), ("k", shards_k), ("v", shards_v)):
        send = [cp.ulysses_pack(s, P, cp.SEQ_TO_HEAD) for s in shards]        # [B, P, S_l, Hp, D]
        recv[name] = alltoall(send)                                          # chunk g from rank g
    o_send = []
    for r in range(P):
        B, _, S_l, Hp, D = recv["q"][r].shape
        q, k, v = (recv[n][r].view(B, P * S_l, Hp, D) for n in ("q", "k", "v"))   # [B, S, Hp, D]
        o = torch.empty((B, P, S_l, Hp, D), dtype=torch.bfloat16, device="cuda")
        n = cp.attn_fwd_workspace_size(B, Hp, P * S_l, P * S_l, D) if use_ws else 0
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        cp.attn_fwd_ex(q, k, v, o=o.view(B, P * S_l, Hp, D), workspace=ws, seq_major=True)
        o_send.append(o)                                                     # chunk p -> rank p
    o_recv = alltoall(o_send)                                                # chunk g = heads of rank g
    return [cp.ulysses_unpack(x, P, cp.HEAD_TO_SEQ) for x in o_recv]         # [B, S_l, H, D]


def test_ulysses_fused_small():
    B, H, P, S_l, D = 1, 8, 4, 300, 128
    S = P * S_l
    qb = inputs.random_bf16((B, S, H, D), 4300)
    kb = inputs.random_bf16((B, S, H, D), 4301)
    vb = inputs.random_bf16((B, S, H, D), 4302)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    sh = lambda t: [t[:, r * S_l:(r + 1) * S_l].contiguous() for r in range(P)]
    o_shards = ulysses_fused(sh(q), sh(k), sh(v), P)
    torch.cuda.synchronize()
    o = torch.cat(o_shards, dim=1)                                           # [B, S, H, D]
    # equals sequence-major attention over the whole sequence, bit for bit (same tiles per head)
    o_ref, _ = cp.attn_fwd_ex(q, k, v, seq_major=True)
    torch.cuda.synchronize()
    assert same_bits(o, o_ref)
    tr = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    O, _ = oracle.attention(f64_of_bf16(tr(qb)), f64_of_bf16(tr(kb)), f64_of_bf16(tr(vb)), scale_of(D))
    err = np.abs(host64(o.transpose(1, 2)) - O)
    log(f"  fused Ulysses vs oracle: O max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


KT_SHAPES = [
    (1, 3, 300, 328, 128),    # ragged Q tail; 5 full key blocks + 8 keys
    (2, 2, 513, 704, 64),     # batch 2, D = 64, 11 full blocks
    (1, 4, 17, 2992, 128),    # the text-token count (46 blocks + 48 keys)
    (1, 2, 256, 8, 128),      # one partial block of 8 keys
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_f32", [False, True], ids=["o_16", "o_f32"])
@pytest.mark.parametrize("B,H,Sq,Skv,D", KT_SHAPES)
def test_k_seq_last_equals_head_major(B, H, Sq, Skv, D, out_f32, dtype):
    """K given as [B, H, D, Skv] (sequence last, the sample's hint-file layout) runs the same
    arithmetic on the same tiles as K [B, H, Skv, D]: the same bits, and the oracle's result."""
    log(f"case: K sequence-last B{B} H{H} Sq{Sq} Skv{Skv} D{D} {dtype} out_f32={out_f32}")
    seed = 4400 + Sq + Skv + D
    qb = inputs.random_bf16((B, H, Sq, D), seed)
    kb = inputs.random_bf16((B, H, Skv, D), seed + 1)
    vb = inputs.random_bf16((B, H, Skv, D), seed + 2)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    if dtype == "f16":
        q, k, v = (x.float().half() for x in (q, k, v))
    od = torch.float32 if out_f32 else None
    o_ref, l_ref = cp.attn_fwd_ex(q, k, v, out_dtype=od)
    kt = k.transpose(2, 3).contiguous()
    o, l = cp.attn_fwd_ex(q, kt, v, out_dtype=od, k_seq_last=True)
    torch.cuda.synchronize()
    assert same_bits(o, o_ref) and same_bits(l, l_ref)
    if dtype == "bf16":
        O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
        assert_bf16_parity(host64(o), host64(l), O, L, "K sequence-last")


def test_k_seq_last_split_and_accumulate():
    """The key-range split and the accumulate epilogue with K sequence-last: chunks of keys folded
    into one f32 accumulator, each call with its planned workspace, equal the head-major fold bit
    for bit and the oracle over all keys."""
    B, H, Sq, D = 1, 2, 1000, 128
    edges = [0, 1504, 1512, 3000]
    qb = inputs.random_bf16((B, H, Sq, D), 4500)
    kb = inputs.random_bf16((B, H, edges[-1], D), 4501)
    vb = inputs.random_bf16((B, H, edges[-1], D), 4502)
    q = dev_bf16(qb)
    outs = {}
    for kt_layout in (False, True):
        o = torch.empty((B, H, Sq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, Sq), device="cuda")
        for i, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
            k = dev_bf16(np.ascontiguousarray(kb[:, :, a:b]))
            v = dev_bf16(np.ascontiguousarray(vb[:, :, a:b]))
            n = cp.attn_fwd_workspace_size(B, H, Sq, b - a, D, o_dtype=1)
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
            if kt_layout:
                k = k.transpose(2, 3).contiguous()
            cp.attn_fwd_ex(q, k, v, o=o, lse=lse, workspace=ws, accumulate=i > 0, k_seq_last=kt_layout)
        outs[kt_layout] = (o, lse)
    torch.cuda.synchronize()
    assert same_bits(outs[True][0], outs[False][0]) and same_bits(outs[True][1], outs[False][1])
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(outs[True][0]), host64(outs[True][1]), O, L, "K sequence-last folded")


def test_k_seq_last_many_units():
    """Enough tiles for the dynamic schedule's per-XCD ranges and its tail, and a split of the
    last wave: K sequence-last equals K head-major bit for bit (outputs pre-filled with NaN)."""
    B, H, Sq, Skv, D = 1, 24, 5520, 2992, 128
    qb = inputs.random_bf16((B, H, Sq, D), 4600)
    kb = inputs.random_bf16((B, H, Skv, D), 4601)
    vb = inputs.random_bf16((B, H, Skv, D), 4602)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = cp.attn_fwd_ex(q, k, v, workspace=ws)
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    cp.attn_fwd_ex(q, k.transpose(2, 3).contiguous(), v, o=o, lse=l, workspace=ws, k_seq_last=True)
    torch.cuda.synchronize()
    assert same_bits(o, o_ref) and same_bits(l, l_ref)
