// Non-causal attention forward with 8-bit float inputs (OCP FP8 E4M3) on gfx950's
// v_mfma_f32_32x32x64_f8f6f4 (twice the bf16 matrix-core rate).
//
// Same method as the bf16 kernel (blockwise online softmax, "Scaling AI inference
// across multiple GPUs using NVIDIA TensorRT with multi-device inference support",
// section "Ring Attention"; low-precision inference named in its opening section):
// Q, K, V arrive as E4M3 bytes with one f32 scale per tensor, scores and softmax
// state are f32, the softmax weights are rounded to E4M3 for the PV product, and O
// is stored as bf16 or f32.  D = 128.
//
// Work split and schedule follow the bf16 kernel: 8 waves, 256 query rows per
// workgroup, waves w and w+4 on one SIMD alternating an MFMA slot (4 QK + 4 PV MFMAs
// per 64-key block) with a softmax slot, K/V through four LDS buffers by direct
// global->LDS loads issued inside the MFMA slot three blocks ahead, Q^T in registers.
// The softmax slot is the critical one here (its exponentials, at one wave's VALU
// issue rate, outlast the MFMA slot, whose length is set by the 16 KB of LDS operands
// a wave reads per block), so it issues no loads and the MFMA slot takes over the row
// max of the block it has just multiplied, between its PV MFMAs.
//
// Operand layouts of the 32x32x64 fp8 MFMA: lane (row/column l%32, half h = l/32)
// holds 32 bytes of its row of A (column of B); byte j of half h of A meets byte j
// of half h of B.  QK: both operands hold d = 64*ks + 32*h + j.  PV: the B operand
// is P^T straight from the S^T accumulator, whose lane (query, h) holds accumulator
// rows (i/4)*8 + 4h + i%4 of each 32-key tile.  K rows are stored in LDS with bits 2
// and 3 of the row index swapped, so that accumulator row rho holds the key
// rho ^ swap23, and half h's bytes 8c..8c+7 are the 8 consecutive keys 16c + 8h + e.
// The V^T A operand then comes from four ds_read_b64_tr_b8 per MFMA: in each 16-lane
// group, lane pair (2i, 2i+1) addresses row r0 + i (bytes 0-7 and 8-15 of a 16-byte
// column block) and lane L receives column L of the 8 rows.
//
// Rows are 128 bytes; 16-byte chunks are XOR-swizzled by a permutation of the row pair
// (swz8 below) so that both the K reads (16 rows x one chunk) and the transposing V reads
// (8 rows x two chunks per 32 lanes) hit distinct banks.
//
// Softmax: t = s * c with c = scale * log2(e) * q_scale * k_scale; the running max is
// raised only when a block's max exceeds it by more than 1, so p = exp2(t - m) <= 2;
// the weights enter the PV product as E4M3 of p * 2^7 (<= 256 < 448, and typical
// weights stay in E4M3's normal range), computed directly as exp2(t - m + 7); the row
// sum l' of these unrounded f32 values carries the same 2^7, so O = sum(p8 v) * v_scale
// / l' and LSE = (m + log2 l' - 7) * ln 2.
#include <climits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "unit_sched.h"

#define CPATTN_AI __attribute__((always_inline))

namespace cpattn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define GLOBAL_PTR(T, p) ((const __attribute__((address_space(1))) T*)(p))

template <int I>
using ic = std::integral_constant<int, I>;

constexpr int kD = 128;
constexpr int kBM = kAttnTileRows;   // 256 query rows per workgroup
constexpr int kBN = 64;              // keys per block
constexpr int kNBUF = 4;
constexpr float kRaiseTh = 1.0f;     // raise m only when a block max exceeds it by more than 1
constexpr float kPScaleLog2 = 7.0f;  // p enters the PV product as E4M3(p * 2^7)

// Stored 16-byte chunk of logical chunk c of row r is c ^ swz8(r), with swz8 a permutation of
// the row pair u = (r >> 1) & 7: u -> ((u & 3) << 1) | (u >> 2).  K reads (16 consecutive rows,
// one chunk): the 8 row pairs take 8 distinct values.  Transposing V reads (per 32 lanes: 8
// consecutive rows 8m..8m+7 x the two chunks 2dt, 2dt+1): the four row pairs take values of
// distinct s >> 1, so the chunk pairs {2dt ^ s, (2dt + 1) ^ s} are disjoint.  Both hit 64
// distinct banks.
__device__ __forceinline__ int swz8(int r) {
    const int u = (r >> 1) & 7;
    return ((u & 3) << 1) | (u >> 2);
}
// LDS row of K that holds key (row) r of the block, and back: swap bits 2 and 3
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// two f32 -> two E4M3 bytes in the low (HI=false) or high half of `old`, nearest even
template <bool HI>
__device__ __forceinline__ int pack_fp8x2(float a, float b, int old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// One work unit of a workgroup: a whole query tile k_unit < map.n_dp, or a key-range piece
// (numbering, piece bounds and the dynamic-schedule claim as in the 16-bit kernel: a piece leaves
// its normalised f32 O and natural LSE in the workspace for the piece merge).
template <bool OUT_F32, bool SEQ>
__device__ __forceinline__ int attn_unit_fp8(int k_unit, const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                                             const uint8_t* __restrict__ v, void* __restrict__ o,
                                             float* __restrict__ lse, int Sq, int Skv_all, int nQt, int H, Strides sq,
                                             Strides skv, Strides so, AttnTileMap map, float c, float v_scale,
                                             int* next_lds) {
    constexpr int D = kD, BN = kBN;
    constexpr int NKS = D / 64;            // k-steps of QK (64 d each)
    constexpr int NDT = D / 32;            // 32-wide d tiles of O^T
    constexpr int NKT = BN / 32;           // 32-key tiles of S^T
    constexpr int RPP = 1024 / D;          // rows per 1 KB load piece (8)

    __shared__ __attribute__((aligned(1024))) uint8_t Ks[kNBUF][BN * D];
    __shared__ __attribute__((aligned(1024))) uint8_t Vs[kNBUF][BN * D];

    const int nblk_all = (Skv_all + BN - 1) / BN;
    int tile, kb0 = 0, slot = -1, nblk = nblk_all;
    if (k_unit < map.n_dp) {
        tile = k_unit;
    } else {
        const int logical = k_unit - map.n_dp;
        const int p = logical / map.n_split;
        const int ti = logical - p * map.n_split;
        tile = map.n_dp + ti;
        slot = ti * map.split_s + p;
        kb0 = (int)((int64_t)p * nblk_all / map.split_s);
        nblk = (int)((int64_t)(p + 1) * nblk_all / map.split_s) - kb0;
    }
    const int Skv = min(Skv_all - kb0 * BN, nblk * BN);   // keys of this unit
    const int bh = tile / nQt;
    const int qt = tile - bh * nQt;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int L16 = lane & 15;
    const int g16 = (lane >> 4) & 1;
    const int group = wave >> 2;

    const int64_t q_row = SEQ ? sq.row : D, kv_row = SEQ ? skv.row : D, o_row = SEQ ? so.row : D;
    const int b = SEQ ? bh / H : 0, h = SEQ ? bh - b * H : 0;
    const int64_t kv_off =
        (SEQ ? b * skv.batch + h * skv.head : (int64_t)bh * Skv_all * D) + (int64_t)kb0 * BN * kv_row;
    const uint8_t* qp = q + (SEQ ? b * sq.batch + h * sq.head : (int64_t)bh * Sq * D);
    const uint8_t* kp = k + kv_off;
    const uint8_t* vp = v + kv_off;
    const int64_t o_base = SEQ ? b * so.batch + h * so.head : (int64_t)bh * Sq * D;
    const int qrow = qt * kBM + wave * 32 + l32;

    // One 1 KB piece per wave per tensor: LDS rows 8*wave .. 8*wave+7 of the block.  A load is
    // the block's wave-uniform base (SGPRs) plus a per-lane byte offset that is the same for
    // every full block; the last, partial block clamps its rows.  M0 holds the LDS base;
    // nothing else in this kernel uses M0, so the asm sets it itself.
    const int lrow = wave_u * RPP + lane / 8;                         // LDS row of this lane
    const int lch = (lane % 8) ^ swz8(lrow);                          // logical chunk it moves
    const uint32_t koffb = (uint32_t)(swap23(lrow) * kv_row + lch * 16);   // K row swap23(lrow)
    const uint32_t voffb = (uint32_t)(lrow * kv_row + lch * 16);
    auto load_block = [&](const uint8_t* src, uint8_t* dst, int j, bool is_k) CPATTN_AI {
        const uint32_t lds = (uint32_t)(uintptr_t)LDS_PTR(void, dst + wave_u * 1024);
        const uint8_t* blk = src + (int64_t)j * BN * kv_row;
        uint32_t off;
        if ((j + 1) * BN <= Skv) {
            off = is_k ? koffb : voffb;
        } else {
            const int key = min(is_k ? swap23(lrow) : lrow, Skv - 1 - j * BN);
            off = (uint32_t)(key * kv_row + lch * 16);
        }
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0"
                     :: "v"(off), "s"(blk), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
    };

    // Q^T operand: lane (query l32, half hh), k-step ks: bytes d = 64 ks + 32 hh .. +31
    i32x8 qreg[NKS];
    {
        const uint8_t* qr = qp + min(qrow, Sq - 1) * q_row + 32 * hh;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(qr + 64 * ks);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(qr + 64 * ks + 16);
            qreg[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                             (int)hi[3]};
        }
    }
    // K operand of tile kt, k-step ks: LDS row 32 kt + l32, logical chunks 4 ks + 2 hh, +1
    auto read_k = [&]<int BUF>(ic<BUF>, int kt, int ks) CPATTN_AI -> i32x8 {
        const int row = kt * 32 + l32;
        const uint8_t* base = &Ks[BUF][row * D];
        const int c0 = 4 * ks + 2 * hh;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + ((c0 ^ swz8(row)) * 16));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (((c0 + 1) ^ swz8(row)) * 16));
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // V^T operand of d tile dt: four transposing reads, rows 16 c + 8 hh + (L16 / 2), chunk of
    // columns dt*32 + 16 g16 .. +15, bytes 8 (L16 % 2) of it
    auto read_vt = [&]<int BUF>(ic<BUF>, int dt) CPATTN_AI -> i32x8 {
        i32x2 r[4];
        const int lchunk = dt * 2 + g16;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int row = 16 * cc + 8 * hh + (L16 >> 1);
            r[cc] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                LDS_PTR(i32x2, &Vs[BUF][row * D + ((lchunk ^ swz8(row)) * 16) + 8 * (L16 & 1)]));
        }
        return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    };

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    f32x16 s[NKT];
    i32x8 pb = {0, 0, 0, 0, 0, 0, 0, 0};   // P^T bytes: j = 16 kt + i
    float m_run = -INFINITY, l_run = 0.f, alpha = 1.f;

    // Loads for block j, issued inside M_j: this wave's pieces of K_{j+3} and V_{j+2}, into the
    // buffers of K_{j-1} and V_{j-2}, which M_{j-1} of both groups finished reading before the
    // previous barrier.  The softmax slot, the critical one here, issues none.
    // FULL: the caller guarantees K_{j+3} and V_{j+2} exist and are full blocks (no runtime
    // check, so no branch in the MFMA stream)
    auto dma_full = [&](const uint8_t* src, uint8_t* dst, int j, uint32_t off) CPATTN_AI {
        const uint32_t lds = (uint32_t)(uintptr_t)LDS_PTR(void, dst + wave_u * 1024);
        const uint8_t* blk = src + (int64_t)j * BN * kv_row;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0"
                     :: "v"(off), "s"(blk), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
    };
    auto issue_k = [&]<int R, bool FULL>(ic<R>, std::bool_constant<FULL>, int j) CPATTN_AI {
        if constexpr (FULL) dma_full(kp, Ks[(R + 3) % 4], j + 3, koffb);
        else if (j + 3 < nblk) load_block(kp, Ks[(R + 3) % 4], j + 3, true);
    };
    auto issue_v = [&]<int R, bool FULL>(ic<R>, std::bool_constant<FULL>, int j) CPATTN_AI {
        if constexpr (FULL) dma_full(vp, Vs[(R + 2) % 4], j + 2, voffb);
        else if (j + 2 < nblk) load_block(vp, Vs[(R + 2) % 4], j + 2, false);
    };
    // Row max of S_j (keys past Skv in the last block first set to -inf), in two halves so
    // that each follows a PV MFMA, then the lazy raise of the running max and alpha.
    float mx_part = -INFINITY;
    bool raise = false;
    auto row_max_half = [&]<bool FULL>(int kt, std::bool_constant<FULL>, int j) CPATTN_AI {
        if (!FULL && kt == 0 && j == nblk - 1 && (Skv % BN) != 0) {
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j * BN + swap23(t * 32 + (i >> 2) * 8 + hh * 4 + (i & 3));
                    if (key >= Skv) s[t][i] = -INFINITY;
                }
        }
        float mx = kt == 0 ? s[0][0] : mx_part;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
        mx_part = mx;
    };
    auto raise_max = [&]() CPATTN_AI {
        const float mx = max_across_halves(mx_part) * c;
        raise = mx > m_run + kRaiseTh;
        const float m_new = raise ? mx : m_run;
        alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
    };
    // M_j: S_j = K_j Q^T (j < nblk) and O += V_{j-1} P_{j-1} (j >= 1), then the row max of
    // S_j; R = j % 4.  Every operand of the slot is read from LDS up front, so no MFMA waits
    // on a read issued just before it.
    auto M = [&]<int R, bool QK, bool PV, bool FULL>(ic<R>, std::bool_constant<QK>, std::bool_constant<PV>,
                                                   std::bool_constant<FULL>, int j) CPATTN_AI {
        constexpr int KB = R, VB = (R + 3) % 4;
        __builtin_amdgcn_s_setprio(1);
        i32x8 kf[NKS * NKT], vf[NDT];
        if constexpr (QK) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) kf[ks * NKT + kt] = read_k(ic<KB>{}, kt, ks);
        }
        if constexpr (PV) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) vf[dt] = read_vt(ic<VB>{}, dt);
        }
        if constexpr (QK) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    s[kt] = mfma8(kf[ks * NKT + kt], qreg[ks], s[kt]);
                    if (ks == 0 && kt == 1) {
                        __builtin_amdgcn_sched_barrier(0);
                        issue_k(ic<R>{}, std::bool_constant<FULL>{}, j);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PV) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                oacc[dt] = mfma8(vf[dt], pb, oacc[dt]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (QK) {
                    if (dt == 0) row_max_half(0, std::bool_constant<FULL>{}, j);
                    if (dt == 1) {
                        issue_v(ic<R>{}, std::bool_constant<FULL>{}, j);
                        __builtin_amdgcn_sched_barrier(0);
                        row_max_half(1, std::bool_constant<FULL>{}, j);
                        raise_max();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else if constexpr (QK) {
            issue_v(ic<R>{}, std::bool_constant<FULL>{}, j);
            row_max_half(0, std::bool_constant<FULL>{}, j);
            row_max_half(1, std::bool_constant<FULL>{}, j);
            raise_max();
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // SM_j: P_j (E4M3 of p * 2^7) from S_j and the running max, the row sum, O *= alpha when
    // some row raised its max
    auto SM = [&]() CPATTN_AI {
        // every weight reads m_run: tying it here keeps this work after the slot barrier
        // (the barrier orders memory only, and the max is already known before it)
        asm volatile("" : "+v"(m_run));
        const float mb = kPScaleLog2 - m_run;   // weights come out scaled by 2^7
        // Every exponent argument of the block first, then every exponential, then the row sum
        // (four independent partial sums, no serial chain of dependent adds) and the packs, kept
        // apart by scheduling fences so that no instruction waits on the one just before it.
#pragma unroll
        for (int x = 0; x < NKT * 16; ++x) s[x / 16][x % 16] = __builtin_fmaf(s[x / 16][x % 16], c, mb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < NKT * 16; ++x) s[x / 16][x % 16] = exp2_fast(s[x / 16][x % 16]);
        __builtin_amdgcn_sched_barrier(0);
        float psum[4];
#pragma unroll
        for (int x = 0; x < NKT * 16; ++x) {
            if (x < 4) psum[x] = s[0][x];
            else psum[x & 3] += s[x / 16][x % 16];
        }
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // both halves of the word are written, so the previous contents are irrelevant
                int word = pack_fp8x2<false>(s[kt][w * 4 + 0], s[kt][w * 4 + 1], pb[kt * 4 + w]);
                word = pack_fp8x2<true>(s[kt][w * 4 + 2], s[kt][w * 4 + 3], word);
                pb[kt * 4 + w] = word;
            }
        l_run = l_run * alpha + ((psum[0] + psum[1]) + (psum[2] + psum[3]));
        asm volatile("" : "+v"(l_run));
        asm volatile("" : "+v"(pb));
        if (__ballot(raise) != 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
        }
    };
    // wait until at most this wave's latest issue (two loads when full) is in flight: then
    // the blocks issued in M_{j-2} are complete before the barrier ahead of slot 2j+1
    auto wait_older = [&]<bool FULL>(std::bool_constant<FULL>, int jl) CPATTN_AI {
        if (FULL || jl + 3 < nblk) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    load_block(kp, Ks[0], 0, true);
    if (nblk > 1) load_block(kp, Ks[1], 1, true);
    if (nblk > 2) load_block(kp, Ks[2], 2, true);
    load_block(vp, Vs[0], 0, false);
    if (nblk > 1) load_block(vp, Vs[1], 1, false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Both groups run M_0, SM_0, ..., M_nblk; group 1 one slot behind (an extra barrier up
    // front; group 0 adds one at the end).
    auto slot_barrier = [&]() CPATTN_AI { asm volatile("s_barrier" ::: "memory"); };
    auto body = [&]<int R, bool QK, bool PV, bool FULL = false>(ic<R>, std::bool_constant<QK>, std::bool_constant<PV>,
                                                              int j, std::bool_constant<FULL> = {}) CPATTN_AI {
        M(ic<R>{}, std::bool_constant<QK>{}, std::bool_constant<PV>{}, std::bool_constant<FULL>{}, j);
        __builtin_amdgcn_sched_barrier(0);
        wait_older(std::bool_constant<FULL>{}, j);
        __builtin_amdgcn_sched_barrier(0);
        slot_barrier();
        if constexpr (QK) SM();
        wait_older(std::bool_constant<FULL>{}, j);
        __builtin_amdgcn_sched_barrier(0);
        slot_barrier();
    };
    using T = std::true_type;
    using F = std::false_type;
    if (group != 0) slot_barrier();
    body(ic<0>{}, T{}, F{}, 0);
    int j = 1;
    // steady state with no runtime checks: every load of these four blocks is a full block
    // and none of them is the last block (each check removed is a branch in the slots)
    const int nfull = Skv / BN;
    for (; j + 7 <= nfull; j += 4) {
        body(ic<1>{}, T{}, T{}, j, T{});
        body(ic<2>{}, T{}, T{}, j + 1, T{});
        body(ic<3>{}, T{}, T{}, j + 2, T{});
        body(ic<0>{}, T{}, T{}, j + 3, T{});
    }
    // Dynamic schedule: claim the next unit now, a few blocks before the end, so that the
    // atomic's round trip overlaps the last blocks (it is complete by the end of the next
    // softmax slot, and its result is first read after the epilogue).
    unsigned long long claim = 0;
    if (map.sched != nullptr && tid == 0) claim = sched_ticket(map, k_unit, (int)blockIdx.x);
    for (; j + 3 < nblk; j += 4) {
        body(ic<1>{}, T{}, T{}, j);
        body(ic<2>{}, T{}, T{}, j + 1);
        body(ic<3>{}, T{}, T{}, j + 2);
        body(ic<0>{}, T{}, T{}, j + 3);
    }
    if (j < nblk) body(ic<1>{}, T{}, T{}, j);
    if (j + 1 < nblk) body(ic<2>{}, T{}, T{}, j + 1);
    if (j + 2 < nblk) body(ic<3>{}, T{}, T{}, j + 2);
    switch (nblk & 3) {      // M_nblk: the last PV product only
        case 0: body(ic<0>{}, F{}, T{}, nblk); break;
        case 1: body(ic<1>{}, F{}, T{}, nblk); break;
        case 2: body(ic<2>{}, F{}, T{}, nblk); break;
        default: body(ic<3>{}, F{}, T{}, nblk); break;
    }
    if (group == 0) slot_barrier();

    // epilogue: l carries the 2^7 of the weights; O = acc * v_scale / l, LSE natural
    const float l_tot = sum_across_halves(l_run);
    const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
    const float lse_new = l_tot > 0.f ? (m_run + log2f(l_tot) - kPScaleLog2) * kLn2 : -INFINITY;
    if (slot >= 0) {
        const size_t wrow = (size_t)slot * kBM + wave * 32 + l32;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = dt * 32 + g * 8 + hh * 4;
                *reinterpret_cast<f32x4*>(map.ws_o + wrow * D + d0) =
                    f32x4{oacc[dt][g * 4 + 0] * inv, oacc[dt][g * 4 + 1] * inv, oacc[dt][g * 4 + 2] * inv,
                          oacc[dt][g * 4 + 3] * inv};
            }
        if (hh == 0) map.ws_lse[wrow] = lse_new;
    } else if (qrow < Sq) {
        const int64_t orow = o_base + qrow * o_row;
        float wa = 0.f, wb = inv, L = lse_new;   // O = wa * O_old + wb * acc
        // accumulating: every old value is loaded before the first store to the same row
        f32x4 old[OUT_F32 ? NDT * 4 : 1];
        if constexpr (OUT_F32) {
            if (map.accumulate) {
                const float la = lse[(size_t)bh * Sq + qrow];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        old[dt * 4 + g] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + orow +
                                                                          dt * 32 + g * 8 + hh * 4);
                const float mx = fmaxf(la, lse_new);
                wb = 0.f;
                L = -INFINITY;
                if (mx != -INFINITY) {
                    const float ea = expf(la - mx), eb = expf(lse_new - mx);
                    const float tot = ea + eb;
                    L = mx + logf(tot);
                    wa = ea / tot;
                    wb = eb / tot * inv;
                }
            }
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = dt * 32 + g * 8 + hh * 4;
                f32x4 x = f32x4{oacc[dt][g * 4 + 0], oacc[dt][g * 4 + 1], oacc[dt][g * 4 + 2],
                                oacc[dt][g * 4 + 3]} * wb;
                if constexpr (OUT_F32) {
                    if (map.accumulate) x += old[dt * 4 + g] * wa;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow + d0) = x;
                } else {
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + orow + d0) =
                        u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                }
            }
        if (hh == 0) lse[(size_t)bh * Sq + qrow] = L;
    }
    if (map.sched == nullptr) return -1;
    // the claim is first used here, after the epilogue's stores are issued; every wave read the
    // previous one before the first barrier of this unit
    __builtin_amdgcn_sched_barrier(0);
    if (tid == 0) *next_lds = sched_next(map, k_unit, (int)blockIdx.x, (int)gridDim.x, claim);
    __syncthreads();
    return *next_lds;
}

// Persistent workgroups over work units, with the static or the dynamic schedule of the 16-bit
// kernel (see attn_fwd_kernel.h: the first round XCD-aware, later units from the counter).
template <bool OUT_F32, bool SEQ>
__global__ __launch_bounds__(512) void attn_fwd_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                                                           const uint8_t* __restrict__ v, void* __restrict__ o,
                                                           float* __restrict__ lse, int Sq, int Skv, int nQt, int H,
                                                           Strides sq, Strides skv, Strides so, AttnTileMap map,
                                                           float c, float v_scale, int n_grid) {
    __shared__ int next_unit;
    const int n_units = map.n_dp + map.n_split * map.split_s;
    const bool dynamic = map.sched != nullptr;
    const int G = (int)gridDim.x;
    const int bb = (int)blockIdx.x;
    int64_t bid = bb;
    int u;
    if (dynamic) {
        u = sched_first(map, bb);
    } else {
        u = -1;
        for (; bid < n_grid && u < 0; bid += G) u = sched_static_unit(map, bid);
    }
    while (u >= 0 && u < n_units) {       // one call site: the unit body is inlined once
        const int claimed =
            attn_unit_fp8<OUT_F32, SEQ>(u, q, k, v, o, lse, Sq, Skv, nQt, H, sq, skv, so, map, c, v_scale, &next_unit);
        if (dynamic) {
            u = claimed;
        } else {
            u = -1;
            for (; bid < n_grid && u < 0; bid += G) u = sched_static_unit(map, bid);
        }
    }
}


// Clears the dynamic schedule's counters (kSchedWords words) before a launch that uses one.
__global__ void zero_sched_kernel_fp8(unsigned long long* sched) {
    for (int i = threadIdx.x; i < kSchedWords; i += blockDim.x) sched[i] = 0;
}

template <bool OUT_F32, bool SEQ>
hipError_t launch_fp8_typed(const AttnFp8Args& a) {
    const int nQt = (int)((a.Sq + kBM - 1) / kBM);
    const int64_t total = a.BH * nQt;
    const UnitGrid ug = sched_plan(total, a.split_tiles, a.split_pieces, a.slots, a.sched != nullptr);
    AttnTileMap m = ug.map;
    m.ws_o = a.ws_o;
    m.ws_lse = a.ws_lse;
    m.accumulate = a.accumulate ? 1 : 0;
    m.sched = a.sched;
    const int grid = ug.grid, launch_grid = ug.launch_grid;
    const float c = (float)((double)a.scale * 1.4426950408889634 * (double)a.q_scale * (double)a.k_scale);
    if (a.sched != nullptr && a.sched_clear) {
        hipLaunchKernelGGL(zero_sched_kernel_fp8, dim3(1), dim3(256), 0, a.stream, a.sched_clear);
        const hipError_t ez = hipGetLastError();
        if (ez != hipSuccess) return ez;
    }
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<OUT_F32, SEQ>), dim3(launch_grid), dim3(512), 0, a.stream,
                       static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                       static_cast<const uint8_t*>(a.v), a.o, a.lse, (int)a.Sq, (int)a.Skv, nQt, (int)a.H, a.sq,
                       a.skv, a.so, m, c, a.v_scale, grid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_tiles == 0) return e;
    MergePiecesArgs f{a.ws_o, a.ws_lse, a.o, a.lse, m.n_dp, m.n_split, m.split_s, nQt, a.H, a.so, a.Sq, kD,
                      OUT_F32 ? MergeOut::F32 : MergeOut::BF16, a.accumulate, a.stream};
    return launch_merge_pieces(f);
}

template <bool OUT_F32>
int occupancy_fp8() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_fp8_kernel<OUT_F32, false>, 512, 0) != hipSuccess)
        return 0;
    return n;
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const AttnFp8Args& a) {
    if (a.seq_major) return a.out_f32 ? launch_fp8_typed<true, true>(a) : launch_fp8_typed<false, true>(a);
    return a.out_f32 ? launch_fp8_typed<true, false>(a) : launch_fp8_typed<false, false>(a);
}

int attn_fwd_fp8_blocks_per_cu(bool out_f32) { return out_f32 ? occupancy_fp8<true>() : occupancy_fp8<false>(); }

}  // namespace cpattn
