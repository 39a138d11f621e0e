"""GPU Ulysses relayout: bit-exact against the oracle's index maps."""
import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import (assert_bf16_parity, dev_bf16, f64_of_bf16, host64, log, scale_of)

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("B,S_l,H,D,P,dtype", [(1, 5520, 24, 128, 8, "bf16"), (2, 37, 12, 64, 4, "bf16"),
                                               (1, 9, 6, 8, 3, "bf16"), (1, 11, 8, 4, 2, "f32"),
                                               (1, 1, 8, 128, 8, "bf16"),
                                               (1, 7, 6, 72, 3, "bf16"),      # 9 chunks of 16 B per row
                                               (2, 5, 4, 320, 2, "bf16"),     # 40 chunks, tiles of 12 rows
                                               (1, 3, 4, 8192, 2, "bf16")])   # 1024 chunks: a tile per row
def test_relayout_bit_exact(B, S_l, H, D, P, dtype):
    log(f"case: relayout B{B} S_l{S_l} H{H} D{D} P{P} {dtype}")
    rng = np.random.Generator(np.random.PCG64(S_l + H))
    if dtype == "bf16":
        shard = rng.integers(0, 1 << 16, size=(B, S_l, H, D), dtype=np.uint16)   # arbitrary bit patterns
        t = torch.from_numpy(shard.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        shard = rng.integers(-(1 << 31), 1 << 31, size=(B, S_l, H, D), dtype=np.int64).astype(np.int32)
        t = torch.from_numpy(shard).view(torch.float32).cuda()
    send = cp.ulysses_pack(t, P, cp.SEQ_TO_HEAD)
    heads = cp.ulysses_unpack(send, P, cp.SEQ_TO_HEAD)
    send2 = cp.ulysses_pack(heads, P, cp.HEAD_TO_SEQ)
    back = cp.ulysses_unpack(send2, P, cp.HEAD_TO_SEQ)
    torch.cuda.synchronize()
    ref_send = oracle.ulysses_pack(shard, P, oracle.SEQ_TO_HEAD)
    ref_heads = oracle.ulysses_unpack(ref_send, P, oracle.SEQ_TO_HEAD)
    ref_send2 = oracle.ulysses_pack(ref_heads, P, oracle.HEAD_TO_SEQ)
    assert np.array_equal(_bits(send), ref_send)
    assert np.array_equal(_bits(heads), ref_heads)
    assert np.array_equal(_bits(send2), ref_send2)
    assert np.array_equal(_bits(back), shard)


def test_simulated_ulysses_pipeline():
    """8 ranks on one device: pack -> all-to-all (index permutation) -> unpack ->
    attention on each rank's 3 heads -> pack -> all-to-all -> unpack, against
    the oracle's attention over all 24 heads for each rank's tokens."""
    P, S_l, H, D = 8, 96, 24, 128
    S = P * S_l
    g = {n: inputs.random_bf16((1, S, H, D), 300 + i) for i, n in enumerate("qkv")}   # token-major
    shards = {n: [dev_bf16(np.ascontiguousarray(g[n][:, r * S_l:(r + 1) * S_l])) for r in range(P)] for n in "qkv"}

    def a2a(bufs):   # recv[r][:, p] = send[p][:, r]
        return [torch.stack([bufs[p][:, r] for p in range(P)], dim=1).contiguous() for r in range(P)]

    heads = {}
    for n in "qkv":
        recv = a2a([cp.ulysses_pack(shards[n][r], P, cp.SEQ_TO_HEAD) for r in range(P)])
        heads[n] = [cp.ulysses_unpack(recv[r], P, cp.SEQ_TO_HEAD) for r in range(P)]
    outs = [cp.attn_fwd(heads["q"][r], heads["k"][r], heads["v"][r])[0] for r in range(P)]
    recv = a2a([cp.ulysses_pack(outs[r], P, cp.HEAD_TO_SEQ) for r in range(P)])
    back = [cp.ulysses_unpack(recv[r], P, cp.HEAD_TO_SEQ) for r in range(P)]
    torch.cuda.synchronize()
    to_bhsd = lambda x: np.ascontiguousarray(f64_of_bf16(x).transpose(0, 2, 1, 3))
    O, L = oracle.attention(to_bhsd(g["q"]), to_bhsd(g["k"]), to_bhsd(g["v"]), scale_of(D))
    O_tok = O.transpose(0, 2, 1, 3)   # [1, S, H, D]
    got = np.concatenate([host64(b) for b in back], axis=1)
    # LSE is not part of the pipeline's output; compare O only (pass the oracle LSE through)
    assert_bf16_parity(got, L, O_tok, L, "ulysses pipeline")


@pytest.mark.parametrize("n", [1, 3, 8])
@pytest.mark.parametrize("B,S_l,H,D,P", [(1, 5520, 24, 128, 8), (2, 37, 12, 64, 4), (1, 1, 8, 8, 8)])
def test_batched_relayout_bit_exact(B, S_l, H, D, P, n):
    """ulysses_pack_n / ulysses_unpack_n move n tensors in one launch; each result is the
    oracle's index map of its own source, bit for bit, in both directions."""
    log(f"case: batched relayout n={n} B{B} S_l{S_l} H{H} D{D} P{P}")
    rng = np.random.Generator(np.random.PCG64(7000 + n * 100 + S_l))
    shards = [rng.integers(0, 1 << 16, size=(B, S_l, H, D), dtype=np.uint16) for _ in range(n)]
    ts = [torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).cuda() for s in shards]
    send = cp.ulysses_pack_n(ts, P, cp.SEQ_TO_HEAD)
    heads = cp.ulysses_unpack_n(send, P, cp.SEQ_TO_HEAD)
    send2 = cp.ulysses_pack_n(heads, P, cp.HEAD_TO_SEQ)
    back = cp.ulysses_unpack_n(send2, P, cp.HEAD_TO_SEQ)
    torch.cuda.synchronize()
    for i, shard in enumerate(shards):
        ref_send = oracle.ulysses_pack(shard, P, oracle.SEQ_TO_HEAD)
        ref_heads = oracle.ulysses_unpack(ref_send, P, oracle.SEQ_TO_HEAD)
        assert np.array_equal(_bits(send[i]), ref_send), i
        assert np.array_equal(_bits(heads[i]), ref_heads), i
        assert np.array_equal(_bits(send2[i]), oracle.ulysses_pack(ref_heads, P, oracle.HEAD_TO_SEQ)), i
        assert np.array_equal(_bits(back[i]), shard), i
