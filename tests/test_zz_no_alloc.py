"""cpattn_attn_fwd_ex_static, the entry point that allocates nothing, against cpattn_attn_fwd_ex.

Collected last on purpose, so that a failure here cannot hide the other GPU tests.

Both run the same kernels and the same split plan when the static variant may use as many
scratch bytes as the caller's workspace holds, so the outputs must be the same bits.  Two
calls in a row share the device's scratch; the second one is smaller.
"""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import assert_bf16_parity, dev_bf16, f64_of_bf16, host64, log, scale_of

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    v = torch.int16 if a.element_size() == 2 else torch.int32
    return torch.equal(a.contiguous().view(v), b.contiguous().view(v))


def plan_bytes(B, H, Sq, Skv, D, o_dtype):
    return min(cp.attn_fwd_workspace_size(B, H, Sq, Skv, D, cp.BF16, o_dtype), cp.STATIC_SCRATCH_BYTES)


def test_static_scratch_two_calls():
    # call 1: a ring chunk's shape, 24 heads x 5520 rows x 5520 keys; its best plan (16 tiles x 16
    # pieces, 33.8 MB) is over the 32 MiB scratch, so both calls plan within 32 MiB
    B, H, S, D = 1, 24, 5520, 128
    log(f"case: static scratch call 1 [{B},{H},{S},{D}] x {S} keys, bf16 O")
    qb, kb, vb = (inputs.random_bf16((B, H, S, D), 9100 + i) for i in range(3))
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    n1 = plan_bytes(B, H, S, S, D, cp.BF16)
    assert 0 < n1 <= cp.STATIC_SCRATCH_BYTES
    ws = torch.empty(n1, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = cp.attn_fwd_ex(q, k, v, workspace=ws)
    o = torch.empty_like(o_ref)
    l = torch.empty_like(l_ref)
    cp.attn_fwd_ex_static(q, k, v, o=o, lse=l, scratch_bytes=n1)
    torch.cuda.synchronize()
    log(f"  scratch {n1} B: same bits as attn_fwd_ex {same_bits(o, o_ref) and same_bits(l, l_ref)}")
    assert same_bits(o, o_ref) and same_bits(l, l_ref)
    # sampled rows against the oracle (tile edges, the ragged last tile, random rows)
    rows = inputs.sample_rows(S, n_random=16)
    O, L = oracle.attention_rows(f64_of_bf16(qb[:, :4]), f64_of_bf16(kb[:, :4]), f64_of_bf16(vb[:, :4]),
                                 scale_of(D), rows)
    assert_bf16_parity(host64(o[:, :4, rows]), host64(l[:, :4, rows]), O, L, "static scratch, call 1 (sampled)")

    # call 2, smaller, right after on the same device: sequence-major, two key chunks folded into
    # an f32 (O, LSE) by the accumulate flag, 8 tiles x 11 pieces of scratch
    B, H, Sq, Skv, D = 1, 2, 1000, 3000, 128
    log(f"case: static scratch call 2 [{B},{Sq},{H},{D}] x {Skv} keys, sequence-major, accumulate")
    qb, kb, vb = (inputs.random_bf16((B, H, n, D), 9200 + i) for i, n in enumerate((Sq, Skv, Skv)))
    seq = lambda a: dev_bf16(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    q, k, v = seq(qb), seq(kb), seq(vb)
    half = 1400
    n2 = plan_bytes(B, H, Sq, Skv - half, D, cp.F32)
    assert 0 < n2 < n1
    outs = []
    for static in (False, True):
        o = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda")
        l = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
        cp.attn_fwd_ex(q, k[:, :half].contiguous(), v[:, :half].contiguous(), o=o, lse=l, seq_major=True)
        k2, v2 = k[:, half:].contiguous(), v[:, half:].contiguous()
        if static:
            cp.attn_fwd_ex_static(q, k2, v2, o=o, lse=l, scratch_bytes=n2, accumulate=True, seq_major=True)
        else:
            ws = torch.empty(n2, dtype=torch.uint8, device="cuda")
            cp.attn_fwd_ex(q, k2, v2, o=o, lse=l, workspace=ws, accumulate=True, seq_major=True)
        outs.append((o, l))
    torch.cuda.synchronize()
    (o_ref, l_ref), (o, l) = outs
    log(f"  scratch {n2} B: same bits as attn_fwd_ex {same_bits(o, o_ref) and same_bits(l, l_ref)}")
    assert same_bits(o, o_ref) and same_bits(l, l_ref)
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    assert_bf16_parity(host64(o.transpose(1, 2)), host64(l), O, L, "static scratch, call 2")


def test_static_scratch_refuses_more_than_it_holds():
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cp.CpattnError, match="E_SHAPE"):
        cp.attn_fwd_ex_static(q, q, q, scratch_bytes=cp.STATIC_SCRATCH_BYTES + 1)
    # no scratch at all: the unsplit kernel, as attn_fwd_ex without a workspace
    o, l = cp.attn_fwd_ex_static(q, q, q, scratch_bytes=0)
    o2, l2 = cp.attn_fwd_ex(q, q, q)
    torch.cuda.synchronize()
    assert same_bits(o, o2) and same_bits(l, l2)
