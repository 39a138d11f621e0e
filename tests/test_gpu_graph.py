"""The per-rank path captured into a HIP graph and replayed.

Every launch the library makes goes onto the caller's stream, and clearing the
schedule's work counters is a kernel of its own (not a memset), so the calls can
be recorded into a graph.  One graph holds:

* cpattn_attn_fwd_ex_static on a shape whose query tiles are split into key-range
  pieces (counter clear, attention, piece merge; the static scratch, no allocation);
* cpattn_attn_fwd_ex with a caller workspace and the accumulate flag, folding into
  an f32 (O, LSE) that is reset to its starting values before every replay;
* cpattn_ring_attn_fwd over three K/V chunks with its work buffers;
* cpattn_ulysses_pack of a [S_local, H, D] shard.

The graph is replayed three times, with eager work and synchronisations between the
replays and the outputs overwritten with NaN before each one; every replay must give
the eager calls' results bit for bit.  The eager results are checked against the
oracle here too.
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


def test_graph_replays_match_eager():
    B, H, Sq, Skv, D = 1, 4, 1000, 3000, 128        # 16 tiles on 256 slots, 47 key blocks: split
    n_chunks, Skv_c = 3, 1000
    S_l, P = 1104, 8
    log(f"case: graph capture, attention [{B},{H},{Sq},{D}] x {Skv}, ring {n_chunks} x {Skv_c}, "
        f"pack [{S_l},{H * 6},{D}] P={P}")
    qb = inputs.random_bf16((B, H, Sq, D), 9300)
    kb = inputs.random_bf16((B, H, Skv, D), 9301)
    vb = inputs.random_bf16((B, H, Skv, D), 9302)
    kcb = inputs.random_bf16((n_chunks, B, H, Skv_c, D), 9303)
    vcb = inputs.random_bf16((n_chunks, B, H, Skv_c, D), 9304)
    xb = inputs.random_bf16((B, S_l, H * 6, D), 9305)
    q, k, v, kc, vc, x = (dev_bf16(a) for a in (qb, kb, vb, kcb, vcb, xb))

    n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D)
    tiles, pieces, _ = cp.attn_fwd_split_plan(B, H, Sq, Skv, D, 256, n)
    log(f"  plan for 256 slots: {tiles} tiles x {pieces} pieces")
    assert pieces > 1
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o1 = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device="cuda")
    l1 = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    # the accumulate call folds into the result of a separate key set
    kab, vab = inputs.random_bf16((B, H, 300, D), 9306), inputs.random_bf16((B, H, 300, D), 9307)
    ka, va = dev_bf16(kab), dev_bf16(vab)
    o2_init, l2_init = cp.attn_fwd(q, ka, va, out_dtype=torch.float32)
    o2, l2 = torch.empty_like(o2_init), torch.empty_like(l2_init)
    o3 = torch.empty((B, H, Sq, D), dtype=torch.float32, device="cuda")
    l3 = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    ow, lw = torch.empty_like(o3), torch.empty_like(l3)
    pk = torch.empty((B, P, S_l, H * 6 // P, D), dtype=torch.bfloat16, device="cuda")

    def calls():
        cp.attn_fwd_ex_static(q, k, v, o=o1, lse=l1)
        cp.attn_fwd_ex(q, k, v, o=o2, lse=l2, workspace=ws, accumulate=True)
        cp.ring_attn_fwd(q, kc, vc, o=o3, lse=l3, o_work=ow, lse_work=lw)
        cp.ulysses_pack(x, P, cp.SEQ_TO_HEAD, dst=pk)

    outs = (o1, l1, o2, l2, o3, l3, pk)
    # eager run (it also makes the library's one-time per-device lookups before the capture)
    o2.copy_(o2_init)
    l2.copy_(l2_init)
    calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    q64, k64, v64 = f64_of_bf16(qb), f64_of_bf16(kb), f64_of_bf16(vb)
    O, L = oracle.attention(q64, k64, v64, scale_of(D))
    assert_bf16_parity(host64(ref[0]), host64(ref[1]), O, L, "static entry point, split")
    O, L = oracle.attention(q64, np.concatenate([f64_of_bf16(kab), k64], axis=2),
                            np.concatenate([f64_of_bf16(vab), v64], axis=2), scale_of(D))
    assert_bf16_parity(host64(ref[2]), host64(ref[3]), O, L, "accumulate onto a second key set")
    kcat = np.concatenate([f64_of_bf16(kcb[c]) for c in range(n_chunks)], axis=2)
    vcat = np.concatenate([f64_of_bf16(vcb[c]) for c in range(n_chunks)], axis=2)
    O, L = oracle.attention(q64, kcat, vcat, scale_of(D))
    assert_bf16_parity(host64(ref[4]), host64(ref[5]), O, L, "ring over three chunks")
    assert np.array_equal(ref[6].cpu().view(torch.int16).numpy().view(np.uint16),
                          oracle.ulysses_pack(xb, P, oracle.SEQ_TO_HEAD))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    other = torch.empty_like(o1)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        o2.copy_(o2_init)
        l2.copy_(l2_init)
        cp.attn_fwd(q, ka, va, o=other)          # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = [same_bits(a, b) for a, b in zip(outs, ref)]
        log(f"  replay {rep}: same bits as eager {same}")
        assert all(same), f"replay {rep}"
