// Non-causal attention forward, bf16 inputs, bf16 matrix cores (gfx950).
//
// Computes, per (b, h) and query row i, the online-softmax form of
//   O_i = sum_j softmax_j(scale * q_i . k_j) v_j,   LSE_i = ln sum_j exp(scale * q_i . k_j)
// streaming K/V in blocks of BN rows, as Ring Attention's blockwise online
// softmax does ("Scaling AI inference across multiple GPUs using NVIDIA
// TensorRT with multi-device inference support", section "Ring Attention";
// no causal mask, section "Context parallelism").
//
// Work split.  One workgroup = NWAVES wave64s = one tile of BM = 32*NWAVES
// query rows of one (b, h); wave w owns rows [32w, 32w+32) of the tile.
//
// Transposed formulation.  Each wave computes S^T = K Q^T and O^T = V^T P^T
// with v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane
// holds one column, so with queries on the column axis every lane owns one
// query row: row max and row sum are lane-local apart from one exchange
// between the two 32-lane halves, the softmax weights P^T come out of the
// S^T accumulator already laid out as the B operand of the PV product (no
// LDS round trip for P), and the rescale of O by exp(m_old - m_new) is a
// per-lane scalar.
//
//   S^T tile (32 keys x 32 queries):  lane l, register i holds
//       key   (i/4)*8 + (l/32)*4 + i%4,  query l%32.
//   PV k-step t covers the 16 keys 16t..16t+15 of the block; lane half h
//   supplies slots (h, 0..7) = S^T registers 8*(t%2)..+7 of key tile t/2,
//   i.e. keys 16t + 8*(j/4) + 4h + j%4.  The V^T A-operand must use the same
//   key order, so V is stored in LDS transposed with bits 2 and 3 of the key
//   index swapped; each A fragment is then one 16-byte LDS read.
//
// Staging.  K (row-major, padded) and V^T (padded) blocks live in LDS,
// double-buffered: the global loads for block j+1 are issued before the
// MFMAs of block j and written to the other buffer after them, with one
// workgroup barrier per block.
//
// Softmax in base 2: t = s * scale * log2(e); p = exp2(t - m); the natural
// LSE is (m + log2 l) * ln 2.  Keys past Skv in the last block get -inf.
#include "common.h"
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int BN = 64;     // keys per block
constexpr int KPAD = 8;    // bf16 pad per K row in LDS (keeps 16B reads conflict-free)
constexpr int VPAD = 8;    // bf16 pad per V^T row in LDS

__device__ __forceinline__ int swap_bits23(int x) {
    return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

template <int D, int NWAVES, bool OUT_F32>
__global__ __launch_bounds__(NWAVES * 64) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* __restrict__ o, float* __restrict__ lse, int Sq, int Skv, int nQt, int total_tiles,
    int per_xcd, float c) {
    constexpr int NT = NWAVES * 64;
    constexpr int BM = NWAVES * 32;
    constexpr int KSTR = D + KPAD;
    constexpr int VSTR = BN + VPAD;
    constexpr int NKS = D / 16;             // k-steps of the QK^T product
    constexpr int NDT = D / 32;             // 32-wide d tiles of O^T
    constexpr int KCH = (BN * D / 8 + NT - 1) / NT;   // 16-byte K chunks per thread
    constexpr int NVSB = (BN / 4) * (D / 4);          // 4x4 V sub-blocks per block
    constexpr int VSB = (NVSB + NT - 1) / NT;         // sub-blocks per thread

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VSTR];

    // XCD-aware tile order: workgroup ids dealt round-robin over the XCDs are
    // mapped so that each XCD walks a contiguous range of tiles, i.e. the
    // workgroups resident on one XCD share a head and its K/V stream in L2.
    const int bid = blockIdx.x;
    const int logical = (bid % kNumXcd) * per_xcd + bid / kNumXcd;
    if (logical >= total_tiles) return;
    const int bh = logical / nQt;
    const int qt = logical - bh * nQt;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const uint16_t* qp = q + (size_t)bh * Sq * D;
    const uint16_t* kp = k + (size_t)bh * Skv * D;
    const uint16_t* vp = v + (size_t)bh * Skv * D;
    const int qrow = qt * BM + wave * 32 + l32;

    // Q^T fragments (B operand of S^T = K Q^T): query qrow, dims 16*ks + 8*hh .. +7.
    u32x4 qf[NKS];
    if (qrow < Sq) {
        const u32x4* src = reinterpret_cast<const u32x4*>(qp + (size_t)qrow * D);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = src[2 * ks + hh];
    } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = u32x4{0, 0, 0, 0};
    }

    u32x4 kreg[KCH];
    u32x2 vreg[VSB][4];

    auto load_block = [&](int j) {
        const int kv0 = j * BN;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ch = tid + i * NT;
            const int row = ch / (D / 8);
            const int c8 = ch - row * (D / 8);
            const int kv = kv0 + row;
            if (ch < BN * D / 8 && kv < Skv)
                kreg[i] = reinterpret_cast<const u32x4*>(kp + (size_t)kv * D)[c8];
            else
                kreg[i] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < VSB; ++i) {
            const int sb = tid + i * NT;
            const int dq = (sb & 7) + ((sb >> 3) / (BN / 4)) * 8;
            const int kvq = (sb >> 3) % (BN / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kv = kv0 + kvq * 4 + r;
                if (sb < NVSB && kv < Skv)
                    vreg[i][r] = reinterpret_cast<const u32x2*>(vp + (size_t)kv * D)[dq];
                else
                    vreg[i][r] = u32x2{0, 0};
            }
        }
    };

    auto store_block = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ch = tid + i * NT;
            const int row = ch / (D / 8);
            const int c8 = ch - row * (D / 8);
            if (ch < BN * D / 8)
                *reinterpret_cast<u32x4*>(&Ks[buf][row * KSTR + c8 * 8]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VSB; ++i) {
            const int sb = tid + i * NT;
            if (sb >= NVSB) continue;
            const int dq = (sb & 7) + ((sb >> 3) / (BN / 4)) * 8;
            const int kvq = (sb >> 3) % (BN / 4);
            const int pos = swap_bits23(kvq * 4);
            // vreg[i][r] = V[kv = 4*kvq + r][4*dq .. 4*dq+3] as two dwords (d pairs).
            // Output for d = 4*dq + e: keys r = 0..3 -> two dwords (r0|r1<<16, r2|r3<<16).
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int w = e >> 1;
                const bool hi = e & 1;
                uint32_t a0 = vreg[i][0][w], a1 = vreg[i][1][w], a2 = vreg[i][2][w], a3 = vreg[i][3][w];
                uint32_t lo_pair = hi ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
                uint32_t hi_pair = hi ? ((a2 >> 16) | (a3 & 0xFFFF0000u)) : ((a2 & 0xFFFFu) | (a3 << 16));
                *reinterpret_cast<u32x2*>(&Vt[buf][(dq * 4 + e) * VSTR + pos]) = u32x2{lo_pair, hi_pair};
            }
        }
    };

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;

    float m_run = -INFINITY;   // running max, base-2 units (scale*log2e applied)
    float l_run = 0.f;         // this lane half's partial row sum

    const int nblk = (Skv + BN - 1) / BN;
    load_block(0);
    store_block(0);
    __syncthreads();

    for (int j = 0; j < nblk; ++j) {
        const int buf = j & 1;
        if (j + 1 < nblk) load_block(j + 1);

        // ---- S^T = K Q^T for the 64 keys of this block (two 32-key tiles)
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
            const uint16_t* krow = &Ks[buf][(kt * 32 + l32) * KSTR + hh * 8];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                u32x4 a = *reinterpret_cast<const u32x4*>(krow + ks * 16);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                __builtin_bit_cast(bf16x8, qf[ks]),
                                                                s[kt], 0, 0, 0);
            }
        }

        // ---- mask keys past Skv (only the last block can have them)
        if ((j + 1) * BN > Skv) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j * BN + kt * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
                    if (key >= Skv) s[kt][i] = -INFINITY;
                }
        }

        // ---- online softmax (row = this lane's query)
        float mx = s[0][0];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
        mx = max_across_halves(mx);
        const float m_new = fmaxf(m_run, mx * c);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;

        float psum = 0.f;
        u32x4 pb[4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = exp2_fast(__builtin_fmaf(s[kt][half * 8 + e], c, -m_new));
                    psum += p[e];
                }
                pb[kt * 2 + half] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;

        // ---- O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const uint16_t* vrow = &Vt[buf][(dt * 32 + l32) * VSTR + hh * 8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 a = *reinterpret_cast<const u32x4*>(vrow + t * 16);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                   __builtin_bit_cast(bf16x8, pb[t]),
                                                                   oacc[dt], 0, 0, 0);
            }
        }

        if (j + 1 < nblk) store_block(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O / l, LSE = (m + log2 l) ln 2
    const float l_tot = sum_across_halves(l_run);
    if (qrow < Sq) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        const size_t orow = ((size_t)bh * Sq + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = dt * 32 + g * 8 + hh * 4;
                const float x0 = oacc[dt][g * 4 + 0] * inv, x1 = oacc[dt][g * 4 + 1] * inv;
                const float x2 = oacc[dt][g * 4 + 2] * inv, x3 = oacc[dt][g * 4 + 3] * inv;
                if constexpr (OUT_F32) {
                    *reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow + d0) = f32x4{x0, x1, x2, x3};
                } else {
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + orow + d0) =
                        u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
                }
            }
        if (hh == 0)
            lse[(size_t)bh * Sq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, int NWAVES, bool OUT_F32>
hipError_t launch(const AttnFwdArgs& a) {
    constexpr int BM = NWAVES * 32;
    const int nQt = (int)((a.Sq + BM - 1) / BM);
    const int64_t total = (int64_t)a.BH * nQt;
    const int per_xcd = (int)((total + kNumXcd - 1) / kNumXcd);
    const int grid = per_xcd * kNumXcd;
    const float c = (float)((double)a.scale * 1.4426950408889634);
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NWAVES, OUT_F32>), dim3(grid), dim3(NWAVES * 64), 0,
                       a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.o, a.lse, (int)a.Sq, (int)a.Skv, nQt,
                       (int)total, per_xcd, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a) {
    if (a.D == 128) return a.out_f32 ? launch<128, 8, true>(a) : launch<128, 8, false>(a);
    return a.out_f32 ? launch<64, 8, true>(a) : launch<64, 8, false>(a);
}

}  // namespace cpattn
