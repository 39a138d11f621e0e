"""GPU parity of fp8 (OCP E4M3) attention against the fp64 oracle.

The oracle computes exact attention of the real-valued inputs (decoded E4M3 bytes times
their per-tensor scales).  The kernel keeps scores and softmax state in f32 but rounds
each softmax weight to E4M3 for the PV product, so the tolerance is derived from that
rounding rather than taken from the bf16 gates:

- a weight P_ij (normalised) enters as E4M3 of p * 2^7 with p <= 2 and the row sum >= 1,
  so its error is at most 2^-4 relative (half an ulp of a 3-bit mantissa) or 2^-17
  absolute (half the subnormal step); the fp8 matrix core's own accumulation (about
  1e-4 relative, measured) moves the scores and adds 1e-3 relative;
- the errors of different keys are bounded and independent, so by Hoeffding's
  inequality the error of O_id stays below 7 * sqrt(sum_j (e_ij v_jd)^2), with
  e_ij = max((2^-4 + 1e-3) P_ij, 2^-17), except with probability < 1e-10 per element;
- plus the output rounding (bf16: 2^-8 |O|);
- LSE depends only on the scores: |dLSE| <= scale * 1e-4 * max_j sum_d |q_id k_jd| + 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import _lib, inputs
from helpers import log

pytestmark = pytest.mark.gpu


def dev8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def check_fp8(q8, k8, v8, qs, ks, vs, scale, o, lse, what, out_f32=False, rows=None):
    """Compare (o, lse) [B,H,Sq(,D)] with the oracle on the decoded, scaled inputs."""
    q = oracle.e4m3_to_f64(q8) * qs
    k = oracle.e4m3_to_f64(k8) * ks
    v = oracle.e4m3_to_f64(v8) * vs
    if rows is not None:
        q = q[:, :, rows]
    O, L = oracle.attention(q, k, v, scale)
    og = o.detach().float().cpu().numpy().astype(np.float64)
    lg = lse.detach().cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    err = np.abs(og - O)
    bound = np.zeros_like(O)
    lbound = np.zeros_like(L)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            z = scale * (q[b, h] @ k[b, h].T)
            P = np.exp(z - L[b, h][:, None])
            e = np.maximum((2.0 ** -4 + 1e-3) * P, 2.0 ** -17)
            bound[b, h] = 7.0 * np.sqrt((e ** 2) @ (v[b, h] ** 2))
            lbound[b, h] = scale * 1e-4 * np.max(np.abs(q[b, h]) @ np.abs(k[b, h]).T, axis=1) + 1e-5
    bound += (2.0 ** -24 if out_f32 else 2.0 ** -8) * np.abs(O) + 1e-6
    lerr = np.abs(lg - L)
    log(f"  {what}: O max-abs {err.max():.3e} mean-abs {err.mean():.3e} (max err/bound {np.max(err / bound):.3f}); "
        f"LSE max-abs {lerr.max():.3e} (max err/bound {np.max(lerr / lbound):.3f})")
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    assert np.all(err <= bound), f"{what}: O outside the derived bound"
    assert np.all(lerr <= lbound), f"{what}: LSE outside the derived bound"
    return err


SHAPES = [(1, 2, 300, 333, 128), (1, 3, 513, 3000, 128), (2, 1, 17, 64, 128), (1, 2, 256, 2992, 128)]


@pytest.mark.parametrize("seq_major", [False, True], ids=["bhsd", "bshd"])
@pytest.mark.parametrize("out_f32", [False, True], ids=["o_bf16", "o_f32"])
@pytest.mark.parametrize("B,H,Sq,Skv,D", SHAPES)
def test_fp8_small(B, H, Sq, Skv, D, out_f32, seq_major):
    log(f"case: fp8 B{B} H{H} Sq{Sq} Skv{Skv} D{D} out_f32={out_f32} seq_major={seq_major}")
    seed = 7000 + Sq + Skv
    q8 = inputs.random_e4m3((B, H, Sq, D), seed)
    k8 = inputs.random_e4m3((B, H, Skv, D), seed + 1)
    v8 = inputs.random_e4m3((B, H, Skv, D), seed + 2)
    tr = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))) if seq_major else (lambda a: a)
    scale = 1.0 / math.sqrt(D)
    o, lse = cp.attn_fwd_fp8(dev8(tr(q8)), dev8(tr(k8)), dev8(tr(v8)), scale=scale,
                             out_dtype=torch.float32 if out_f32 else None, seq_major=seq_major)
    torch.cuda.synchronize()
    og = o.transpose(1, 2) if seq_major else o
    check_fp8(q8, k8, v8, 1.0, 1.0, 1.0, scale, og, lse, "fp8", out_f32)


def test_fp8_scales_and_large_scores():
    """Per-tensor scales fold into the scores and the output; large scores (q drawn with
    std 4) exercise the running-max raise with the weights still within E4M3's range."""
    B, H, Sq, Skv, D = 1, 2, 300, 1000, 128
    qs, ks, vs = 0.5, 2.0, 0.25
    q8 = inputs.f32_to_e4m3(inputs.random_f32((B, H, Sq, D), 7100, scale=4.0) / qs)
    k8 = inputs.random_e4m3((B, H, Skv, D), 7101, scale=1.0 / ks)
    v8 = inputs.random_e4m3((B, H, Skv, D), 7102, scale=1.0 / vs)
    scale = 1.0 / math.sqrt(D)
    o, lse = cp.attn_fwd_fp8(dev8(q8), dev8(k8), dev8(v8), qs, ks, vs, scale=scale)
    torch.cuda.synchronize()
    check_fp8(q8, k8, v8, qs, ks, vs, scale, o, lse, "fp8 with scales")


def test_fp8_float8_dtype_and_empty_keys():
    q8 = inputs.random_e4m3((1, 2, 40, 128), 7200)
    q = dev8(q8).view(torch.float8_e4m3fn)
    kv = torch.empty((1, 2, 0, 128), dtype=torch.float8_e4m3fn, device="cuda")
    o = torch.full((1, 2, 40, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 2, 40), device="cuda")
    cp.attn_fwd_fp8(q, kv, kv, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.slow
def test_fp8_video_self_attention_sampled():
    S, H, D = inputs.S_VIDEO, inputs.N_HEADS, inputs.HEAD_DIM
    log("case: fp8 self-attention S=44160 H=24 D=128 (E4M3 of N(0,1) draws)")
    q8 = inputs.random_e4m3((1, H, S, D), 7300)
    k8 = inputs.random_e4m3((1, H, S, D), 7301)
    v8 = inputs.random_e4m3((1, H, S, D), 7302)
    o, lse = cp.attn_fwd_fp8(dev8(q8), dev8(k8), dev8(v8))
    torch.cuda.synchronize()
    rows = inputs.sample_rows(S, n_random=8)
    heads = [0, 11, 23]
    for h in heads:
        err = check_fp8(q8[:, h:h + 1], k8[:, h:h + 1], v8[:, h:h + 1], 1.0, 1.0, 1.0, 1.0 / math.sqrt(D),
                        o[:, h:h + 1], lse[:, h:h + 1], f"fp8 S=44160 head {h}", rows=rows)
        # at this length the bf16 gates hold as well
        assert err.max() <= 2e-2 and err.mean() <= 2e-3


def ws_fp8(B, H, Sq, Skv, D, out_f32):
    n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D, cp.E4M3, cp.F32 if out_f32 else cp.BF16)
    return torch.empty(n, dtype=torch.uint8, device="cuda"), n


@pytest.mark.parametrize("seq_major", [False, True], ids=["bhsd", "bshd"])
@pytest.mark.parametrize("out_f32", [False, True], ids=["o_bf16", "o_f32"])
@pytest.mark.parametrize("B,H,Sq,Skv,D", [(1, 2, 1000, 3000, 128), (1, 3, 513, 1100, 128), (1, 1, 17, 2992, 128)])
def test_fp8_split(B, H, Sq, Skv, D, out_f32, seq_major):
    """With a workspace the last wave's tiles are cut into key-range pieces (each a normalised
    f32 partial with its LSE) and folded by the piece merge; units after the first round come
    from the work counter.  Same derived bound as the unsplit call."""
    log(f"case: fp8 split B{B} H{H} Sq{Sq} Skv{Skv} out_f32={out_f32} seq_major={seq_major}")
    seed = 7400 + Sq + Skv
    q8, k8, v8 = (inputs.random_e4m3(s, seed + i) for i, s in enumerate([(B, H, Sq, D), (B, H, Skv, D),
                                                                          (B, H, Skv, D)]))
    tr = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))) if seq_major else (lambda a: a)
    ws, n = ws_fp8(B, H, Sq, Skv, D, out_f32)
    assert n > _lib.SCHED_BYTES, "the planner was expected to split this shape"
    o, lse = cp.attn_fwd_fp8(dev8(tr(q8)), dev8(tr(k8)), dev8(tr(v8)), out_dtype=torch.float32 if out_f32 else None,
                             seq_major=seq_major, workspace=ws)
    torch.cuda.synchronize()
    check_fp8(q8, k8, v8, 1.0, 1.0, 1.0, 1.0 / math.sqrt(D), o.transpose(1, 2) if seq_major else o, lse,
              "fp8 split", out_f32)


@pytest.mark.parametrize("B,H,Sq,Skv", [(1, 24, 4096, 256), (1, 8, 44160, 200)])
def test_fp8_dynamic_schedule_same_bits(B, H, Sq, Skv):
    """More tiles than resident workgroups, no split: the counter-claimed units run the same
    arithmetic as the static order, so the outputs are the same bits (two calls, one workspace)."""
    log(f"case: fp8 dynamic schedule B{B} H{H} Sq{Sq} Skv{Skv}")
    q, k, v = (dev8(inputs.random_e4m3((B, H, n, 128), 7500 + i)) for i, n in enumerate((Sq, Skv, Skv)))
    ws, n = ws_fp8(B, H, Sq, Skv, 128, False)
    assert n == _lib.SCHED_BYTES
    o_ref, l_ref = cp.attn_fwd_fp8(q, k, v)
    for rep in range(2):
        # outputs start as NaN, so a unit that no workgroup ran would show
        o = torch.full_like(o_ref, float("nan"))
        l = torch.full_like(l_ref, float("nan"))
        cp.attn_fwd_fp8(q, k, v, o=o, lse=l, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(l, l_ref), rep


@pytest.mark.parametrize("use_ws", [False, True], ids=["no_ws", "ws"])
def test_fp8_accumulate_chunks(use_ws):
    """A ring step in fp8: chunks of keys folded into an f32 (O, LSE) by the accumulate epilogue
    (and the piece merge when split) equal attention over all keys within the derived bound;
    folding into the empty result (O = 0, LSE = -inf) gives the plain call's bits."""
    H, Sq, D = 2, 600, 128
    edges = [0, 1000, 1001, 2650]
    q8 = inputs.random_e4m3((1, H, Sq, D), 7600)
    k8 = inputs.random_e4m3((1, H, edges[-1], D), 7601)
    v8 = inputs.random_e4m3((1, H, edges[-1], D), 7602)
    log(f"case: fp8 accumulate over chunks {edges} use_ws={use_ws}")
    q = dev8(q8)
    o = torch.zeros((1, H, Sq, D), dtype=torch.float32, device="cuda")
    lse = torch.full((1, H, Sq), float("-inf"), device="cuda")
    for a, b in zip(edges[:-1], edges[1:]):
        k, v = dev8(np.ascontiguousarray(k8[:, :, a:b])), dev8(np.ascontiguousarray(v8[:, :, a:b]))
        ws = ws_fp8(1, H, Sq, b - a, D, True)[0] if use_ws else None
        if a == 0:
            o_ref, l_ref = cp.attn_fwd_fp8(q, k, v, out_dtype=torch.float32, workspace=ws)
        cp.attn_fwd_fp8(q, k, v, o=o, lse=lse, workspace=ws, accumulate=True)
        if a == 0:
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32)) and torch.equal(lse, l_ref)
    torch.cuda.synchronize()
    check_fp8(q8, k8, v8, 1.0, 1.0, 1.0, 1.0 / math.sqrt(D), o, lse, "fp8 accumulated", out_f32=True)
