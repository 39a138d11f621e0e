"""GPU parity of the attention sample's path: QK-RMSNorm prologue and fp16 attention.

The sample ("TensorRT multi-device attention inference in practice") runs fp16
self-attention on (seq, batch, 32, 128) tensors with an RMSNorm on Q and K and
the 1/sqrt(head_dim) scale split as a fourth root on each.  Checked here:
- the prologue against the oracle (every element within one 16-bit ulp, almost
  all exact: the kernel evaluates the norm in f32, the oracle exactly);
- fp16 attention against the oracle on small shapes, both layouts;
- the full single-device run (S = 56320) and one rank of two under
  AllGather-KV (28160 query rows), on sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import long_sequence_bidirectional_amd as cp
from long_sequence_bidirectional_amd import inputs
from helpers import assert_bf16_parity, host64, log, scale_of

pytestmark = pytest.mark.gpu

# fp16 gates: the required ones (max-abs 2e-2, mean-abs 2e-3 on O) plus diagnostics.  fp16
# keeps 11 significant bits: output rounding is <= 2^-12 relative and the rounding of the
# softmax weights averages out over the keys, so rel-L2 of O stays near 5e-4; LSE comes
# from f32 sums only.
F16_REL_L2 = 2e-3
F16_LSE_MAX_ABS = 1e-4


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def assert_f16_parity(o_gpu, lse_gpu, O, L, what):
    d = np.abs(o_gpu - O)
    rel = float(np.linalg.norm(o_gpu - O) / np.linalg.norm(O))
    lse_err = float(np.max(np.abs(lse_gpu - L)))
    log(f"  {what}: O max-abs {d.max():.3e} mean-abs {d.mean():.3e} rel-L2 {rel:.3e}; LSE max-abs {lse_err:.3e}")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert rel <= F16_REL_L2, rel
    assert lse_err <= F16_LSE_MAX_ABS, lse_err


def ulp16(x, dtype):
    """Spacing of the 16-bit type at |x| (float64)."""
    x = np.abs(np.asarray(x, np.float64))
    if dtype == "f16":
        return np.spacing(x.astype(np.float16)).astype(np.float64)
    return np.ldexp(1.0, np.frexp(x)[1] - 8)


def prologue_bound(x, w, scale, dtype):
    """Largest |kernel - oracle| the prologue allows per element.  The kernel evaluates the
    norm in f32, so its rounded RMSNorm value may sit one 16-bit ulp from the exactly rounded
    one; the scale step maps that to s16 * ulp(intermediate), plus one ulp of the result for
    the second rounding."""
    inter = oracle.qk_prologue(x, w, 1e-6, None, dtype=dtype)
    if scale is None:
        return ulp16(inter, dtype)
    s16 = float(oracle.qk_prologue(np.ones((1, 1)), np.ones(1), 0.0, scale, dtype=dtype)[0, 0])
    final = oracle.qk_prologue(x, w, 1e-6, scale, dtype=dtype)
    return s16 * ulp16(inter, dtype) + ulp16(final, dtype)


def compare_16bit(got, want, bound, what, min_exact=0.999):
    """got, want: arrays of 16-bit values (as float64).  Within bound everywhere, and exact for
    at least min_exact of the elements."""
    d = np.abs(got - want)
    exact = float(np.mean(d == 0))
    log(f"  {what}: exact {exact:.5f}, max |diff| / bound {float(np.max(d / bound)):.2f}")
    assert np.all(d <= bound), f"{what}: a value is outside the bound"
    assert exact >= min_exact, f"{what}: only {exact} exact"


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [128, 64, 8, 512])
@pytest.mark.parametrize("scale", [None, "quarter_root"])
def test_qk_rmsnorm(dtype, D, scale):
    rows = 3000
    x32 = inputs.random_f32((rows, D), 5000 + D, scale=2.0)
    w32 = inputs.random_f32((D,), 5001 + D)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    x = torch.from_numpy(x32).to(tdt).cuda()
    w = torch.from_numpy(w32).to(tdt).cuda()
    s = D ** -0.25 if scale else 1.0
    y = cp.qk_rmsnorm(x, w, 1e-6, s)
    torch.cuda.synchronize()
    xs, ws_ = to_f64(x), to_f64(w)
    sc = s if scale else None
    want = oracle.qk_prologue(xs, ws_, 1e-6, sc, dtype=dtype)
    compare_16bit(to_f64(y), want, prologue_bound(xs, ws_, sc, dtype), f"qk_rmsnorm {dtype} D{D} scale={scale}")


def test_qk_rmsnorm_in_place_and_tiny_rows():
    x = torch.from_numpy(inputs.random_f16((5, 128), 5100)).cuda()     # fewer rows than one wave holds
    w = torch.from_numpy(inputs.random_f16((128,), 5101)).cuda()
    ref = cp.qk_rmsnorm(x, w, 1e-6, 128 ** -0.25)
    cp.qk_rmsnorm(x, w, 1e-6, 128 ** -0.25, out=x)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), ref.view(torch.int16))
    # a zero row: mean(x^2) = 0, so y = 0 * rsqrt(eps) * w = 0
    z = torch.zeros((2, 64), dtype=torch.float16, device="cuda")
    y = cp.qk_rmsnorm(z, torch.ones(64, dtype=torch.float16, device="cuda"), 1e-6)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


SMALL = [(1, 3, 300, 333, 128), (1, 2, 513, 3000, 128), (2, 2, 100, 700, 64)]


@pytest.mark.parametrize("seq_major", [False, True], ids=["bhsd", "bshd"])
@pytest.mark.parametrize("out_f32", [False, True], ids=["o_f16", "o_f32"])
@pytest.mark.parametrize("B,H,Sq,Skv,D", SMALL)
def test_f16_attention(B, H, Sq, Skv, D, out_f32, seq_major):
    log(f"case: f16 attention B{B} H{H} Sq{Sq} Skv{Skv} D{D} out_f32={out_f32} seq_major={seq_major}")
    seed = 5200 + Sq + Skv + D
    q, k, v = (inputs.random_f16(s, seed + i) for i, s in enumerate([(B, H, Sq, D), (B, H, Skv, D), (B, H, Skv, D)]))
    tr = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))) if seq_major else (lambda a: a)
    n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D, cp.F16, cp.F32 if out_f32 else cp.F16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o, lse = cp.attn_fwd_ex(dev16(tr(q)), dev16(tr(k)), dev16(tr(v)), out_dtype=torch.float32 if out_f32 else None,
                            workspace=ws, seq_major=seq_major)
    torch.cuda.synchronize()
    assert o.dtype == (torch.float32 if out_f32 else torch.float16)
    og = to_f64(o.transpose(1, 2) if seq_major else o)
    O, L = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale_of(D))
    assert_f16_parity(og, to_f64(lse), O, L, "f16 attention")


def test_f16_merge_and_accumulate():
    """fp16 O through the standalone merge and the accumulate epilogue."""
    H, Sq, D = 2, 400, 128
    q = inputs.random_f16((1, H, Sq, D), 5300)
    k = inputs.random_f16((1, H, 1100, D), 5301)
    v = inputs.random_f16((1, H, 1100, D), 5302)
    O, L = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale_of(D))
    qd = dev16(q)
    halves = [(dev16(k[:, :, a:b]), dev16(v[:, :, a:b])) for a, b in ((0, 600), (600, 1100))]
    (oa, la), (ob, lb) = (cp.attn_fwd(qd, kk, vv) for kk, vv in halves)
    om, lm = cp.attn_merge(oa, la, ob, lb)
    acc = torch.empty((1, H, Sq, D), dtype=torch.float32, device="cuda")
    lacc = torch.empty((1, H, Sq), device="cuda")
    cp.attn_fwd_ex(qd, *halves[0], o=acc, lse=lacc)
    cp.attn_fwd_ex(qd, *halves[1], o=acc, lse=lacc, accumulate=True)
    torch.cuda.synchronize()
    assert om.dtype == torch.float16
    assert_bf16_parity(to_f64(om), to_f64(lm), O, L, "f16 halves merged")
    assert_f16_parity(to_f64(acc), to_f64(lacc), O, L, "f16 accumulated into f32")


# ------------------------------------------------------------------ the sample at full size
S, HP, D = inputs.P4_SEQ, inputs.P4_HEADS, inputs.HEAD_DIM
S_RANK = S // inputs.P4_RANKS
QSCALE = D ** -0.25


@pytest.fixture(scope="module")
def p4():
    log("generating the attention sample's inputs [1, 56320, 32, 128] fp16")
    return inputs.p4_set()


@pytest.fixture(scope="module")
def p4_dev(p4):
    d = {n: dev16(a) for n, a in p4.items()}
    qn = cp.qk_rmsnorm(d["q"], d["w_q"], 1e-6, QSCALE)
    kn = cp.qk_rmsnorm(d["k"], d["w_k"], 1e-6, QSCALE)
    torch.cuda.synchronize()
    d["qn"], d["kn"] = qn, kn
    return d


HEADS = [0, 13, 31]


def oracle_prologue(p4, name, w, h, rows=None, bound=False):
    x = p4[name][0, :, h] if rows is None else p4[name][0, rows, h]
    args = (x.astype(np.float64), p4[w].astype(np.float64))
    if bound:
        return prologue_bound(*args, QSCALE, "f16")
    return oracle.qk_prologue(*args, 1e-6, QSCALE)


@pytest.mark.slow
def test_p4_prologue_full(p4, p4_dev):
    for h in HEADS:
        for name, w in (("k", "w_k"), ("q", "w_q")):
            compare_16bit(to_f64(p4_dev[name + "n"][0, :, h]), oracle_prologue(p4, name, w, h),
                          oracle_prologue(p4, name, w, h, bound=True), f"{name.upper()} prologue head {h}")


def attention_ws(q, k, v):
    B, Sq, H, Dd = q.shape
    n = cp.attn_fwd_workspace_size(B, H, Sq, k.shape[1], Dd, cp.F16, cp.F16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    return cp.attn_fwd_ex(q, k, v, scale=1.0, workspace=ws, seq_major=True)


@pytest.mark.slow
def test_p4_single_device_and_rank(p4, p4_dev):
    log("case: attention sample, single device S=56320, and rank 0 of 2 (28160 query rows)")
    o_full, l_full = attention_ws(p4_dev["qn"], p4_dev["kn"], p4_dev["v"])
    q_rank = p4_dev["qn"][:, :S_RANK].contiguous()
    o_rank, l_rank = attention_ws(q_rank, p4_dev["kn"], p4_dev["v"])
    torch.cuda.synchronize()
    rows = inputs.sample_rows(S, n_random=12, extra=(S_RANK - 1, S_RANK))
    for h in HEADS:
        kn = oracle_prologue(p4, "k", "w_k", h)[None, None]
        vv = p4["v"][0, :, h].astype(np.float64)[None, None]
        qn = oracle_prologue(p4, "q", "w_q", h, rows)[None, None]
        O, L = oracle.attention(qn, kn, vv, 1.0)
        got_o = to_f64(o_full[0, rows, h])[None, None]
        got_l = to_f64(l_full[0, h, rows])[None, None]
        assert_f16_parity(got_o, got_l, O, L, f"single device, head {h}")
        rr = rows[rows < S_RANK]
        assert_f16_parity(to_f64(o_rank[0, rr, h])[None, None], to_f64(l_rank[0, h, rr])[None, None],
                          O[:, :, :len(rr)], L[:, :, :len(rr)], f"rank 0 of 2, head {h}")
    # whole tiles run the same arithmetic: heads 0-29 of the rank's rows are unsplit in both plans
    assert torch.equal(o_rank[:, :, :30].view(torch.int16), o_full[:, :S_RANK, :30].view(torch.int16))
    d = torch.abs(o_rank.float() - o_full[:, :S_RANK].float()).max().item()
    log(f"  rank 0 vs single device rows 0..28159: O max-abs {d:.3e}")
    assert d <= 2e-2
