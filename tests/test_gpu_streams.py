"""Calls on different streams running at the same time.

include/cpattn.h allows calls on different streams to run concurrently as long as
their buffers do not overlap.  The attention kernels are persistent (at most one
workgroup per resident slot, each looping over units) and the dynamic schedule only
claims units from counters in each call's own workspace, so two calls that share the
GPU must still each run every unit exactly once.  Here a split self-attention, a
ring-driver call and a relayout are enqueued on three streams without any ordering
between them, and each result must equal the same call run alone, bit for bit.
"""
import numpy as np
import pytest
import torch

import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import dev_bf16, log

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    v = torch.int16 if a.element_size() == 2 else torch.int32
    return torch.equal(a.contiguous().view(v), b.contiguous().view(v))


def test_three_streams_match_sequential():
    B, H, Sq, Skv, D = 1, 6, 4000, 3000, 128          # 96 tiles, split into key-range pieces
    n_chunks, Skv_c = 4, 1500
    log(f"case: streams, attention [{B},{H},{Sq},{D}] x {Skv}, ring {n_chunks} x {Skv_c}, pack [5520,24,128]")
    q, k, v = (dev_bf16(inputs.random_bf16(s, 9400 + i)) for i, s in
               enumerate([(B, H, Sq, D), (B, H, Skv, D), (B, H, Skv, D)]))
    qr = dev_bf16(inputs.random_bf16((B, H, 2000, D), 9410))
    kc = dev_bf16(inputs.random_bf16((n_chunks, B, H, Skv_c, D), 9411))
    vc = dev_bf16(inputs.random_bf16((n_chunks, B, H, Skv_c, D), 9412))
    x = dev_bf16(inputs.random_bf16((1, 5520, 24, D), 9413))
    ws = torch.empty(cp.attn_fwd_workspace_size(B, H, Sq, Skv, D), dtype=torch.uint8, device="cuda")
    o1, l1 = torch.empty_like(q), torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    o2 = torch.empty((B, H, 2000, D), dtype=torch.float32, device="cuda")
    l2 = torch.empty((B, H, 2000), dtype=torch.float32, device="cuda")
    ow, lw = torch.empty_like(o2), torch.empty_like(l2)
    pk = torch.empty((1, 8, 5520, 3, D), dtype=torch.bfloat16, device="cuda")

    def run(s1, s2, s3):
        cp.attn_fwd_ex(q, k, v, o=o1, lse=l1, workspace=ws, stream=s1)
        cp.ring_attn_fwd(qr, kc, vc, o=o2, lse=l2, o_work=ow, lse_work=lw, stream=s2)
        cp.ulysses_pack(x, 8, cp.SEQ_TO_HEAD, dst=pk, stream=s3)

    main = torch.cuda.current_stream()
    run(main, main, main)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o1, l1, o2, l2, pk)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        for t in (o1, l1, o2, l2, pk):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        run(*streams)
        torch.cuda.synchronize()
        same = [same_bits(a, b) for a, b in zip((o1, l1, o2, l2, pk), ref)]
        log(f"  concurrent run {rep}: same bits as sequential {same}")
        assert all(same), f"run {rep}"
