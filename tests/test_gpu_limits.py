"""Attention at sizes whose element offsets pass 2^31 (64-bit addressing in every kernel).

Checked through closed forms so the oracle stays cheap:
- keys and values made of one seeded block of keys repeated R times give the
  same O as the block alone, with LSE larger by ln R (each weight appears R
  times, so the softmax is unchanged and the sum of exponentials scales by R);
- queries made of a repeated block of rows give repeated output rows, bit for
  bit when the repeat length is a multiple of the 256-row tile.
Both operand layouts run; K/V offsets reach 23 * 2^27 elements (about 3.1e9)
head-major and 2^20 * 3072 sequence-major.  The relayout and the merge are
checked the same way: a pack followed by the inverse unpack is the identity,
and merging a partial result with itself keeps O and adds ln 2 to the LSE.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import _lib, inputs
from helpers import assert_bf16_parity, dev_bf16, f64_of_bf16, host64, log, scale_of

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

H, D = 24, 128
BLOCK = 16384
REPEAT = 64          # 2^20 keys per head


@pytest.mark.parametrize("seq_major", [False, True], ids=["bhsd", "bshd"])
def test_kv_beyond_2_31_elements(seq_major):
    Sq, Skv = 300, BLOCK * REPEAT
    log(f"case: K/V of {H} x {Skv} x {D} bf16 ({H * Skv * D / 2**31:.1f} x 2^31 elements), seq_major={seq_major}")
    qb = inputs.random_bf16((1, H, Sq, D), 6000)
    kb = inputs.random_bf16((1, H, BLOCK, D), 6001)
    vb = inputs.random_bf16((1, H, BLOCK, D), 6002)
    q = dev_bf16(qb)
    k = dev_bf16(kb).repeat(1, 1, REPEAT, 1)
    v = dev_bf16(vb).repeat(1, 1, REPEAT, 1)
    if seq_major:
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    torch.cuda.synchronize()
    n = cp.attn_fwd_workspace_size(1, H, Sq, Skv, D)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o, lse = cp.attn_fwd_ex(q, k, v, workspace=ws, seq_major=seq_major)
    torch.cuda.synchronize()
    del k, v
    O, L = oracle.attention(f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    og = host64(o.transpose(1, 2) if seq_major else o)
    assert_bf16_parity(og, host64(lse), O, L + math.log(REPEAT), "repeated keys")


def test_q_beyond_2_31_elements():
    Sq, Skv = BLOCK * REPEAT, 2992
    log(f"case: Q of {H} x {Sq} x {D} bf16, O the same ({H * Sq * D / 2**31:.1f} x 2^31 elements)")
    qb = inputs.random_bf16((1, H, BLOCK, D), 6100)
    kb = inputs.random_bf16((1, H, Skv, D), 6101)
    vb = inputs.random_bf16((1, H, Skv, D), 6102)
    q = dev_bf16(qb).repeat(1, 1, REPEAT, 1)
    n = cp.attn_fwd_workspace_size(1, H, Sq, Skv, D)
    assert n == _lib.SCHED_BYTES        # 24 * 4096 tiles fill whole waves: no split, only the schedule counters
    k, v = dev_bf16(kb), dev_bf16(vb)
    o, lse = cp.attn_fwd(q, k, v)
    # the dynamic schedule (counters in the workspace) over the same 98304 units: the same bits
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o2, lse2 = cp.attn_fwd_ex(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(lse2, lse)
    del q, o2, lse2
    # the last block of rows (offsets up to ~3.2e9 elements) repeats the first bit for bit
    last = slice(Sq - BLOCK, Sq)
    assert torch.equal(o[:, :, last].view(torch.int16), o[:, :, :BLOCK].view(torch.int16))
    assert torch.equal(lse[:, :, last], lse[:, :, :BLOCK])
    rows = np.array([0, 255, 256, 5000, BLOCK - 1])
    O, L = oracle.attention(f64_of_bf16(qb[:, :, rows]), f64_of_bf16(kb), f64_of_bf16(vb), scale_of(D))
    far = rows + Sq - BLOCK
    assert_bf16_parity(host64(o[:, :, far]), host64(lse[:, :, far]), O, L, "last rows of a 2^20-row Q")


def test_relayout_beyond_2_31_elements():
    """pack (seq->head) then unpack (head->seq) of the packed buffer is the identity:
    out[s, g*Hp + h] = packed[g, s, h] = src[s, g*Hp + h]."""
    S_l, P = BLOCK * REPEAT, 8
    log(f"case: relayout round trip of a [1, {S_l}, {H}, {D}] bf16 shard ({S_l * H * D / 2**31:.1f} x 2^31 elements)")
    src = dev_bf16(inputs.random_bf16((1, BLOCK, H, D), 6200)).repeat(1, REPEAT, 1, 1)
    src[:, -1] = dev_bf16(inputs.random_bf16((1, 1, H, D), 6201))[:, 0]      # a distinct last token
    packed = cp.ulysses_pack(src, P, cp.SEQ_TO_HEAD)
    back = cp.ulysses_unpack(packed, P, cp.HEAD_TO_SEQ)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), src.view(torch.int16))
    # spot-check the packed layout far past 2^31 elements: chunk p holds heads p*Hp..p*Hp+Hp-1
    Hp = H // P
    assert torch.equal(packed[0, P - 1, S_l - 1].view(torch.int16), src[0, S_l - 1, H - Hp:].view(torch.int16))


def test_merge_beyond_2_31_elements():
    """Merging a partial result with itself keeps O (weights 1/2 each, exact in f32) and adds
    ln 2 to the LSE."""
    S = BLOCK * REPEAT
    log(f"case: merge of f32 O [1, {H}, {S}, {D}] ({H * S * D / 2**31:.1f} x 2^31 elements)")
    o_blk = torch.from_numpy(inputs.random_f32((1, H, BLOCK, D), 6300)).cuda()
    l_blk = torch.from_numpy(inputs.random_f32((1, H, BLOCK), 6301)).cuda()
    o = o_blk.repeat(1, 1, REPEAT, 1)
    lse = l_blk.repeat(1, 1, REPEAT)
    om, lm = cp.attn_merge(o, lse, o, lse)
    torch.cuda.synchronize()
    assert torch.equal(om, o)
    d = torch.max(torch.abs(lm.double() - (lse.double() + math.log(2.0)))).item()
    log(f"  LSE vs LSE + ln 2: max-abs {d:.2e}")
    assert d <= 1e-6 * (1 + torch.max(torch.abs(lse)).item())
