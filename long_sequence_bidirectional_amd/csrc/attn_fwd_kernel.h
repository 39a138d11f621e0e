// Non-causal attention forward on the 16-bit matrix cores of gfx950 (bf16 or fp16 inputs).
//
// Kernel template shared by the bf16 and fp16 instantiation units.
//
// Computes, per (b, h) and query row i, the online-softmax form of
//   O_i = sum_j softmax_j(scale * q_i . k_j) v_j,   LSE_i = ln sum_j exp(scale * q_i . k_j)
// streaming K/V in blocks of BN keys, as Ring Attention's blockwise online
// softmax does ("Scaling AI inference across multiple GPUs using NVIDIA
// TensorRT with multi-device inference support", section "Ring Attention";
// no causal mask, section "Context parallelism").
//
// Work split.  One workgroup = 8 wave64s = one tile of 256 query rows of one
// (b, h); wave w owns rows [32w, 32w+32) of the tile.
//
// Transposed formulation.  Each wave computes S^T = K Q^T and O^T = V^T P^T
// with v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane
// holds one column, so with queries on the column axis every lane owns one
// query row: the row max is lane-local apart from one exchange between the
// two 32-lane halves, the row sum needs no exchange until the epilogue, the
// softmax weights P^T come out of the S^T accumulator already laid out as the
// B operand of the PV product (no LDS round trip for P), and the rescale of O
// is a per-lane scalar.
//
//   S^T tile (32 keys x 32 queries):  lane l, register i holds
//       key (i/4)*8 + (l/32)*4 + i%4,  query l%32.
//   PV k-step t covers the 16 keys 16t..16t+15 of the block; lane half h
//   supplies slots (h, 0..7) = S^T registers 8*(t%2)..+7 of key tile t/2,
//   i.e. keys 16t + 8*(j/4) + 4h + j%4.
//
// Registers and LDS.  Each wave keeps its Q^T operand (32 rows x D) in
// registers for the whole tile.  K and V blocks (four buffers each, 128 KB) are
// stored in LDS row-major with 16-byte chunks XOR-swizzled per row and filled by
// direct global->LDS loads (global_load_lds_dwordx4: lane i writes bytes
// 16i..16i+15 of a 1 KB piece, so a wave's load is a plain copy and needs no
// registers).  A load is the block's wave-uniform base (SGPRs) plus a per-lane
// byte offset that is the same for every full block, so no address arithmetic
// runs per block and no register that a load in flight still has to read is
// rewritten.  The V^T A-operand of the PV product comes from two
// ds_read_b64_tr_b16 per MFMA: in each 16-lane group, lane L points at row
// kv0 + L/4, columns d0 + 4(L%4) .. +3 and receives V[kv0 .. kv0+3][d0 + L],
// i.e. four keys of one head-dim column -- exactly the per-lane k-slots above.
// The swizzles make the K reads (16 rows x one chunk) and the V transposing
// reads (4 rows x 4 chunks) hit 64 distinct banks.  With K stored sequence-last
// ([D, keys] per head) a K block is a [D][64] tile instead, and its fragments
// come from two transposing reads each, which give every lane the same values
// as the row-major tile.
//
// Schedule.  Per key block j a wave runs an MFMA slot M_j = {S_j = K_j Q^T,
// O += V_{j-1} P_{j-1}} and a softmax slot SM_j (max, exp2, row sum, bf16
// weights, rescale of O when needed).  Waves w and w+4 share a SIMD; group 1
// (waves 4-7) runs one slot behind group 0, so on every SIMD one wave issues
// MFMAs while the other computes exponentials, with one workgroup barrier
// per slot.  Two measured limits shape the slots:
//  - a wave's LDS reads return at about 32 bytes per clock, so the MFMA slot
//    (1 KB of operands per MFMA) cannot hide all of them behind its MFMAs.
//    The softmax slot therefore reads the first 8 K fragments of the wave's
//    next MFMA slot into registers, and the MFMA slot reads the rest four
//    MFMAs ahead;
//  - a CU's vector-memory path accepts one 1 KB global->LDS load per ~32
//    clocks and a wave stalls at issue until its loads are taken.  A softmax
//    slot that issued all its loads would stall on the critical path, so each
//    wave issues three of its four pieces inside its MFMA slot, spread between
//    MFMAs, and the fourth at the end of its softmax slot, where it would
//    otherwise wait at the barrier; loads run three blocks ahead of use (four
//    buffers).
// Slot barriers are plain s_barrier: each wave waits only for its own older
// loads (vmcnt) before arriving.  The steady state of the block loop carries no
// runtime checks (it runs while every load of its four blocks is a full block):
// a per-block check costs a compare and, in the common case, a taken scalar
// branch in the MFMA or softmax stream, which the schedule pays far above its
// instruction count.  Workgroups are persistent: at most one per resident slot,
// each looping over work units, so a finished unit is followed by the next one
// without a new workgroup launch.
//
// Softmax in base 2: t = s * scale * log2(e), p = exp2(t - m), natural
// LSE = (m + log2 l) * ln 2.  The running max m is only raised when a block's
// max exceeds it by more than 8 (base-2 units, a factor of 2^8, so p <= 256);
// otherwise the stale m is kept and O needs no rescale.  The result is exact
// after the final division by l because every term of O and l carries the same
// factor 2^-m.  Keys past Skv in the last block get -inf.  A lane whose query
// row lies past Sq loads row Sq - 1 instead, so it computes that row's result
// and stores the same bits there again.
#pragma once

#include <climits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "unit_sched.h"

#ifndef CPATTN_AI
#define CPATTN_AI __attribute__((always_inline))
#endif

namespace cpattn {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define GLOBAL_PTR(T, p) ((const __attribute__((address_space(1))) T*)(p))

constexpr int kBM = kAttnTileRows;    // query rows per workgroup (8 waves x 32)
constexpr int kBN = 64;               // keys per block
constexpr int kReadAhead = 4;         // MFMA operand reads issued this many MFMAs ahead
constexpr int NBUF = 4;               // K and V buffers in LDS
constexpr float kRescaleTh = 8.0f;    // raise m only when the block max exceeds it by > 2^8

template <int I>
using ic = std::integral_constant<int, I>;

// Chunk c of row r is stored at chunk position c ^ swz(r).
template <int D>
__device__ __forceinline__ int swz_k(int r) {     // K and Q: 16 consecutive rows, same chunk
    constexpr int RPB = 256 / (2 * D);            // rows per 256-byte bank row
    return (r / RPB) % (D / 8);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {     // V: 4 consecutive rows x 4 chunks
    constexpr int RPB = 256 / (2 * D);
    return 4 * ((r / RPB) % (D / 32));
}
// K with the sequence last ([D, keys] per head): the LDS tile holds D rows of one 64-key
// block (128 bytes each, two per 256-byte bank row); a transposing read covers 4 consecutive
// rows x 4 chunks, so rows r and r + 2 take opposite halves of the row's 8 chunks.
__device__ __forceinline__ int swz_kt(int r) { return ((r >> 1) & 1) << 2; }

// One v_mfma_f32_32x32x16 of the input type: D(32x32) += A(32x16) B(16x32).
template <bool F16>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

// Two fp32 -> one packed pair of the input type, round to nearest even.
template <bool F16>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) {
    if constexpr (F16) return pack_f16x2(lo, hi);
    else return pack_bf16x2(lo, hi);
}

// One work unit (a whole tile or a key-range piece of one) of a workgroup.  Units are numbered
// k = 0 .. n_dp - 1 for the whole tiles [0, n_dp) and k = n_dp + p * n_split + ti for piece p
// of split tile n_dp + ti (piece-major, so that pieces running together read the same keys).
// A piece p of s covers key blocks [p*nblk/s, (p+1)*nblk/s) and leaves a normalised f32 partial
// and its LSE in workspace slot ti * s + p.
//
// With a dynamic schedule (map.sched) the lane that claims work takes the next unit from the
// counter a few blocks before the end of this one, so the atomic's latency overlaps the last
// blocks; the claim is passed to every wave through *next_lds after the epilogue and returned
// (-1 without a dynamic schedule).
template <int D, bool F16, bool OUT_F32, bool SEQ, bool KT>
__device__ __forceinline__ int attn_unit(
    int k_unit, bool first, int static_next, u32x4 (&qreg)[D / 16], const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, void* __restrict__ o, float* __restrict__ lse,
    int Sq, int Skv_all, int nQt, int H, Strides sq, Strides skv, Strides so, AttnTileMap map, float c,
    int* next_lds) {
    constexpr int BN = kBN;
    constexpr int NC = D / 8;               // 16-byte chunks per row
    constexpr int NKS = D / 16;             // k-steps of the QK^T product
    constexpr int NDT = D / 32;             // 32-wide d tiles of O^T
    constexpr int NKT = BN / 32;            // 32-key tiles of S^T per block
    constexpr int NPB = BN / 16;            // 16-key k-steps of the PV product
    constexpr int BLK_BYTES = BN * D * 2;
    constexpr int LOADS_PER_WAVE = BLK_BYTES / 1024 / 8;
    constexpr int ROWS_PER_LOAD = 1024 / (2 * D);
    constexpr int NQK = NKT * NKS;          // MFMA jobs of S = K Q^T
    constexpr int NPV = NDT * NPB;          // MFMA jobs of O += V^T P^T
    static_assert(LOADS_PER_WAVE >= 1, "block too small for the loader");

    __shared__ __attribute__((aligned(1024))) uint16_t Ks[NBUF][BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs[NBUF][BN * D];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int L16 = lane & 15;
    const int g16 = (lane >> 4) & 1;
    const int group = wave >> 2;            // waves w and w+4 share a SIMD

    // Row strides: D for head-major operands (compile time), runtime for sequence-major ones.
    // KT: K is [D, keys] per head (sequence last; Q, V and O head-major): a block of keys is
    // a column range, block j starting j * BN elements in, its rows Skv_all elements apart.
    const int64_t q_row = SEQ ? sq.row : D, kv_row = SEQ ? skv.row : D, o_row = SEQ ? so.row : D;
    const int64_t kt_row = Skv_all;                   // (KT) row stride of K
    const int64_t k_blk = KT ? (int64_t)BN : (int64_t)BN * kv_row;   // elements from block j to j+1

    // Where a work unit's data lives: its query tile, key range and output rows.
    struct Geom {
        const uint16_t* qp;
        const uint16_t* kp;
        const uint16_t* vp;
        int64_t o_base;
        int bh, qrow, row0, Skv, nblk, slot;      // row0: the tile's first query row
    };
    auto geom = [&](int ku) CPATTN_AI -> Geom {
        const int nblk_all = (Skv_all + BN - 1) / BN;
        int tile, kb0 = 0, slot = -1, nb = nblk_all;
        if (ku < map.n_dp) {
            tile = ku;
        } else {
            const int logical = ku - map.n_dp;
            const int p = logical / map.n_split;
            const int ti = logical - p * map.n_split;
            tile = map.n_dp + ti;
            slot = ti * map.split_s + p;
            kb0 = (int)((int64_t)p * nblk_all / map.split_s);
            nb = (int)((int64_t)(p + 1) * nblk_all / map.split_s) - kb0;
        }
        const int bh = tile / nQt;
        const int qt = tile - bh * nQt;
        const int b = SEQ ? bh / H : 0, h = SEQ ? bh - b * H : 0;
        const int64_t q_base = SEQ ? b * sq.batch + h * sq.head : (int64_t)bh * Sq * D;
        const int64_t kv_head = SEQ ? b * skv.batch + h * skv.head : (int64_t)bh * Skv_all * D;
        Geom g;
        g.qp = q + q_base;
        g.kp = k + kv_head + (int64_t)kb0 * k_blk;
        g.vp = v + kv_head + (int64_t)kb0 * BN * kv_row;
        g.o_base = SEQ ? b * so.batch + h * so.head : (int64_t)bh * Sq * D;
        g.bh = bh;
        g.qrow = qt * kBM + wave * 32 + l32;
        g.row0 = qt * kBM;
        g.Skv = min(Skv_all - kb0 * BN, nb * BN);   // keys of the unit
        g.nblk = nb;
        g.slot = slot;
        return g;
    };
    const Geom cur = geom(k_unit);
    const int Skv = cur.Skv, nblk = cur.nblk, slot = cur.slot, bh = cur.bh, qrow = cur.qrow;
    const int64_t o_base = cur.o_base;
    const uint16_t* kp = cur.kp;
    const uint16_t* vp = cur.vp;

    // ---- direct global -> LDS loads of K/V blocks.  Each wave moves its LOADS_PER_WAVE 1 KB
    // pieces of a block; the per-lane byte offsets within a full block are constant, so a load
    // is the block's (wave-uniform) base in SGPRs plus a fixed VGPR offset and no address
    // arithmetic runs per block.  The last, partial block clamps rows to the last valid one.
    // (KT: a K piece is 8 of the tile's D rows of 128 bytes; lane i fills chunk i % 8 of row i / 8)
    constexpr int KT_NC = BN / 8;           // 16-byte chunks per row of the K^T tile
    uint32_t koffb[LOADS_PER_WAVE], voffb[LOADS_PER_WAVE];
#pragma unroll
    for (int I = 0; I < LOADS_PER_WAVE; ++I) {
        const int row = (wave_u * LOADS_PER_WAVE + I) * ROWS_PER_LOAD + lane / NC;
        if constexpr (KT) {
            const int trow = (wave_u * LOADS_PER_WAVE + I) * (1024 / (2 * BN)) + lane / KT_NC;
            koffb[I] = (uint32_t)(((int64_t)trow * kt_row + (((lane % KT_NC) ^ swz_kt(trow)) * 8)) * 2);
        } else {
            koffb[I] = (uint32_t)((row * kv_row + (((lane % NC) ^ swz_k<D>(row)) * 8)) * 2);
        }
        voffb[I] = (uint32_t)((row * kv_row + (((lane % NC) ^ swz_v<D>(row)) * 8)) * 2);
    }
    // One 1 KB piece: global address sb + off + I*1024 -> LDS lds + I*1024 + 16*lane.  M0 holds
    // the LDS base; nothing else in this kernel uses M0 (no LDS DMA builtins, no indexed
    // register access), so the asm sets it itself.
    auto dma = [&]<int I>(ic<I>, uint32_t off, const char* blk, uint32_t lds) CPATTN_AI {
        const char* sb = blk - I * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
                     :: "v"(off), "s"(sb), "s"(lds), "n"(I * 1024) : "memory", "m0");
#pragma clang diagnostic pop
    };
    // (skv: the unit's key count; the last, partial block clamps its rows to the last key, or
    // with KT its 8-key chunks to the last valid chunk: the key count is a multiple of 8 there)
    auto load_piece = [&]<int I>(ic<I>, const uint16_t* src, uint16_t* dst, int j, bool is_v, int skv_u) CPATTN_AI {
        const uint32_t lds = (uint32_t)(uintptr_t)LDS_PTR(void, dst + wave_u * LOADS_PER_WAVE * 512);
        const char* blk = reinterpret_cast<const char*>(src + (int64_t)j * (is_v ? (int64_t)BN * kv_row : k_blk));
        if ((j + 1) * BN <= skv_u) {
            if (is_v) dma(ic<I>{}, voffb[I], blk, lds);
            else dma(ic<I>{}, koffb[I], blk, lds);
        } else if (KT && !is_v) {
            // the lane fills position lane % 8 of its row, which holds chunk (lane % 8) ^ swz
            const int trow = (wave_u * LOADS_PER_WAVE + I) * (1024 / (2 * BN)) + lane / KT_NC;
            const int ch = min((lane % KT_NC) ^ swz_kt(trow), (skv_u - j * BN) / 8 - 1);
            dma(ic<I>{}, (uint32_t)(((int64_t)trow * kt_row + ch * 8) * 2), blk, lds);
        } else {
            const int row = (wave_u * LOADS_PER_WAVE + I) * ROWS_PER_LOAD + lane / NC;
            const int ch = (lane % NC) ^ (is_v ? swz_v<D>(row) : swz_k<D>(row));
            const int r = min(row, skv_u - 1 - j * BN);
            dma(ic<I>{}, (uint32_t)((r * kv_row + ch * 8) * 2), blk, lds);
        }
    };
    auto load_block = [&](const uint16_t* src, uint16_t* dst, int j, bool is_v, int skv_u) CPATTN_AI {
        [&]<int... Is>(std::integer_sequence<int, Is...>) CPATTN_AI {
            (load_piece(ic<Is>{}, src, dst, j, is_v, skv_u), ...);
        }(std::make_integer_sequence<int, LOADS_PER_WAVE>{});
    };

    // A unit's prologue: its first K/V blocks (K_0..K_2, V_0, V_1) into the LDS buffers of their
    // index, then its Q^T operand into qreg (held for the whole unit: for k-step ks lane (l32, hh)
    // holds q[row l32][16 ks + 8 hh .. +7], rows past Sq clamped to the last valid one).  Issued
    // for the first unit here and for every later unit at the end of the unit before it, once no
    // wave reads the LDS buffers any more, so its latency overlaps that unit's epilogue.
    auto issue_prologue = [&](const Geom& g) CPATTN_AI {
        load_block(g.kp, Ks[0], 0, false, g.Skv);
        if (g.nblk > 1) load_block(g.kp, Ks[1], 1, false, g.Skv);
        if (g.nblk > 2) load_block(g.kp, Ks[2], 2, false, g.Skv);
        load_block(g.vp, Vs[0], 0, true, g.Skv);
        if (g.nblk > 1) load_block(g.vp, Vs[1], 1, true, g.Skv);
        const uint16_t* qr = g.qp + min(g.qrow, Sq - 1) * q_row + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qreg[ks] = *reinterpret_cast<const u32x4*>(qr + 16 * ks);
    };
    // Wait for the prologue.  Vector memory operations complete in issue order and the Q loads
    // are its last ones, so the compiler's wait for qreg (before these empty statements that read
    // it) covers the K/V loads too, yet not the epilogue stores issued after them: the compiler
    // counts those stores and leaves them in flight.  The statements also redefine qreg, so no
    // later use of it waits again (such a wait would also wait for the stores, and for any K/V
    // loads issued since).
    auto wait_prologue = [&]() CPATTN_AI {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(qreg[ks]));
    };

    // ---- LDS read addresses: lane-dependent parts (elements); the rest folds into offsets
    int koff[KT ? 1 : NKS], voff[NDT], kofft[KT ? NKT : 1];
    if constexpr (KT) {
        // K^T tile, transposing reads: lane (L16, g16, hh) addresses row 16 ks + 8 hh + 4 h2 +
        // L16 / 4 and columns (keys) 32 kt + 16 g16 + 4 (L16 % 4) .. + 3, and receives rows
        // r0 .. r0 + 3 of column 32 kt + l32: four consecutive head-dim values of its key, so two
        // reads give the same 8 values per lane as the row-major K fragment
        const int rowl = 8 * hh + (L16 >> 2);            // swz_kt depends on bit 1 of the row only
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            const int col = kt * 32 + 16 * g16 + 4 * (L16 & 3);
            kofft[kt] = rowl * BN + (((col >> 3) ^ swz_kt(rowl)) * 8) + (col & 7);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) koff[ks] = l32 * D + (((2 * ks + hh) ^ swz_k<D>(l32)) * 8);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int col = dt * 32 + 16 * g16 + 4 * (L16 & 3);
        const int row = 4 * hh + (L16 >> 2);
        voff[dt] = row * D + (((col >> 3) ^ swz_v<D>(row)) * 8) + ((col >> 2) & 1) * 4;
    }
    auto read_k = [&]<int BUF>(ic<BUF>, int kt, int ks) CPATTN_AI -> u32x4 {
        if constexpr (KT) {
            i16x4 r[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                r[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(i16x4, &Ks[BUF][(16 * ks + 4 * h2) * BN + kofft[kt]]));
            const u32x2 a0 = __builtin_bit_cast(u32x2, r[0]), a1 = __builtin_bit_cast(u32x2, r[1]);
            return u32x4{a0[0], a0[1], a1[0], a1[1]};
        } else {
            return *reinterpret_cast<const u32x4*>(&Ks[BUF][kt * 32 * D + koff[ks]]);
        }
    };
    auto read_vt = [&]<int BUF>(ic<BUF>, int dt, int t) CPATTN_AI -> u32x4 {
        i16x4 r[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            r[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                LDS_PTR(i16x4, &Vs[BUF][(16 * t + 8 * h2) * D + voff[dt]]));
        const u32x2 a0 = __builtin_bit_cast(u32x2, r[0]), a1 = __builtin_bit_cast(u32x2, r[1]);
        return u32x4{a0[0], a0[1], a1[0], a1[1]};
    };

    // ---- per-wave state
    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    f32x16 s[NKT];             // S_j^T
    u32x4 pb[NPB];             // P_j^T as the B operand of the PV product
    float m_run = -INFINITY;   // running max, base-2 units (scale*log2e applied)
    float l_run = 0.f;         // this lane half's partial row sum
    float alpha = 1.f;

    // MFMA slot body: the job list [QK jobs in (ks, kt) order] ++ [PV jobs in (t, dt)
    // order] (consecutive jobs use different accumulators), operand reads kReadAhead
    // jobs ahead, fenced so the compiler keeps that distance.
    constexpr int NPF = NQK < 8 ? NQK : 8;    // K fragments of the next M slot read in the softmax slot
    u32x4 pre[NPF > 0 ? NPF : 1];
    auto mfma_jobs = [&]<int KB, int VB, bool QK, bool PV, bool USE_PRE>(ic<KB>, ic<VB>, std::bool_constant<QK>,
                                                           std::bool_constant<PV>, std::bool_constant<USE_PRE>, auto&& hook) CPATTN_AI {
        constexpr int J0 = QK ? 0 : NQK;
        constexpr int J1 = PV ? NQK + NPV : NQK;
        constexpr int NJ = J1 - J0;
        if constexpr (QK) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
        }
        u32x4 frag[NJ];
        auto rd = [&]<int I>(ic<I>) CPATTN_AI {
            constexpr int jid = J0 + I;
            if constexpr (USE_PRE && jid < NPF) {
                frag[I] = pre[jid];
            } else if constexpr (jid < NQK) {
                constexpr int kt = jid % NKT, ks = jid / NKT;
                frag[I] = read_k(ic<KB>{}, kt, ks);
            } else {
                constexpr int p = jid - NQK;
                frag[I] = read_vt(ic<VB>{}, p % NDT, p / NDT);
            }
        };
        auto step = [&]<int I>(ic<I>) CPATTN_AI {
            if constexpr (I + kReadAhead < NJ) rd(ic<I + kReadAhead>{});
            constexpr int jid = J0 + I;
            if constexpr (jid < NQK) {
                constexpr int kt = jid % NKT, ks = jid / NKT;
                s[kt] = mfma16<F16>(frag[I], qreg[ks], s[kt]);
            } else {
                constexpr int p = jid - NQK, dt = p % NDT, t = p / NDT;
                oacc[dt] = mfma16<F16>(frag[I], pb[t], oacc[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
            hook(ic<I>{}, ic<NJ>{});
        };
        [&]<int... Is>(std::integer_sequence<int, Is...>) CPATTN_AI {
            (rd(ic<Is>{}), ...);
        }(std::make_integer_sequence<int, (kReadAhead < NJ ? kReadAhead : NJ)>{});
        __builtin_amdgcn_sched_barrier(0);
        [&]<int... Is>(std::integer_sequence<int, Is...>) CPATTN_AI {
            (step(ic<Is>{}), ...);
        }(std::make_integer_sequence<int, NJ>{});
    };
    // Loads issued for block j: this wave's pieces of K_{j+3} and V_{j+2}, into the buffers
    // that M_{j-1} (both groups, slots before the previous barrier) released.  The first
    // NP_M pieces go between the MFMAs of M_j, the last one at the end of SM_j, where the
    // softmax wave would otherwise wait at the barrier.
    constexpr int NP_M = 2 * LOADS_PER_WAVE - 1;
    // FULL: the caller guarantees that K_{j+3} and V_{j+2} exist and are full blocks, so the
    // piece goes out with no runtime check (no branch in the MFMA stream).
    auto issue_part = [&]<int R, int P, bool FULL>(ic<R>, ic<P>, std::bool_constant<FULL>, int j) CPATTN_AI {
        if constexpr (P < LOADS_PER_WAVE) {
            if constexpr (FULL) {
                dma(ic<P>{}, koffb[P], reinterpret_cast<const char*>(kp + (int64_t)(j + 3) * k_blk),
                    (uint32_t)(uintptr_t)LDS_PTR(void, Ks[(R + 3) % 4] + wave_u * LOADS_PER_WAVE * 512));
            } else {
                if (j + 3 < nblk) load_piece(ic<P>{}, kp, Ks[(R + 3) % 4], j + 3, false, Skv);
            }
        } else {
            constexpr int Q = P - LOADS_PER_WAVE;
            if constexpr (FULL) {
                dma(ic<Q>{}, voffb[Q], reinterpret_cast<const char*>(vp + (int64_t)(j + 2) * BN * kv_row),
                    (uint32_t)(uintptr_t)LDS_PTR(void, Vs[(R + 2) % 4] + wave_u * LOADS_PER_WAVE * 512));
            } else {
                if (j + 2 < nblk) load_piece(ic<Q>{}, vp, Vs[(R + 2) % 4], j + 2, true, Skv);
            }
        }
    };
    // M_j: S_j = K_j Q^T (j < nblk) and O += V_{j-1} P_{j-1} (j >= 1); R = j % 4.
    auto M = [&]<int R, bool QK, bool PV, bool USE_PRE, bool FULL>(ic<R>, std::bool_constant<QK>,
                                                                 std::bool_constant<PV>, std::bool_constant<USE_PRE>,
                                                                 std::bool_constant<FULL>, int j) CPATTN_AI {
        constexpr int KB = R, VB = (R + 3) % 4;
        auto hook = [&]<int I, int NJ>(ic<I>, ic<NJ>) CPATTN_AI {
            constexpr int GAP = NJ / NP_M;
            if constexpr (I % GAP == GAP / 2 && I / GAP < NP_M) {
                issue_part(ic<R>{}, ic<I / GAP>{}, std::bool_constant<FULL>{}, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        __builtin_amdgcn_s_setprio(1);
        mfma_jobs(ic<KB>{}, ic<VB>{}, std::bool_constant<QK>{}, std::bool_constant<PV>{}, std::bool_constant<USE_PRE>{}, hook);
        __builtin_amdgcn_s_setprio(0);
    };
    // SM_j: softmax of S_j -> P_j, row statistics, O *= alpha_j when some row raised its max.
    // FULL: block j+1 exists and block j is not the last one.
    auto SM = [&]<int R, bool FULL>(ic<R>, std::bool_constant<FULL>, int j) CPATTN_AI {
        if constexpr (NPF > 0) {
            if (FULL || j + 1 < nblk) {
#pragma unroll
                for (int i = 0; i < NPF; ++i) pre[i] = read_k(ic<(R + 1) % 4>{}, i % NKT, i / NKT);
            }
        }
        if (!FULL && j == nblk - 1 && (Skv % BN) != 0) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j * BN + kt * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
                    if (key >= Skv) s[kt][i] = -INFINITY;
                }
        }
        // Row max and row sum each in four independent partials (no serial chain of dependent
        // instructions through the block).
        float mxp[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = kt == 0 ? 4 : 0; i < 16; ++i) mxp[i & 3] = fmaxf(mxp[i & 3], s[kt][i]);
        float mx = fmaxf(fmaxf(mxp[0], mxp[1]), fmaxf(mxp[2], mxp[3]));
        mx = max_across_halves(mx) * c;
        const bool raise = mx > m_run + kRescaleTh;
        const float m_new = raise ? mx : m_run;
        alpha = exp2_fast(m_run - m_new);   // 1 when not raised; 0 on the first block
        m_run = m_new;
        // Every exponent argument of the block first, then every exponential, then the sums and
        // packs: kept apart by scheduling fences, no instruction waits on the one just before it
        // (measured 1.2-2% faster for the whole kernel than each weight's fma, exp2, add in turn).
#pragma unroll
        for (int x = 0; x < NKT * 16; ++x) s[x / 16][x % 16] = __builtin_fmaf(s[x / 16][x % 16], c, -m_new);
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
            for (int half = 0; half < 2; ++half)
                pb[kt * 2 + half] = u32x4{pack16x2<F16>(s[kt][half * 8 + 0], s[kt][half * 8 + 1]),
                                          pack16x2<F16>(s[kt][half * 8 + 2], s[kt][half * 8 + 3]),
                                          pack16x2<F16>(s[kt][half * 8 + 4], s[kt][half * 8 + 5]),
                                          pack16x2<F16>(s[kt][half * 8 + 6], s[kt][half * 8 + 7])};
        l_run = l_run * alpha + ((psum[0] + psum[1]) + (psum[2] + psum[3]));
        // keep the row sum and the packed weights materialised in this slot (otherwise
        // the compiler defers them past the barrier and holds every weight live)
        asm volatile("" : "+v"(l_run));
#pragma unroll
        for (int t = 0; t < NPB; ++t) asm volatile("" : "+v"(pb[t]));
        if (__builtin_expect(__ballot(raise) != 0, 0)) {   // rare: keep the common path free of taken branches
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
        }
    };
    // Wait until at most this wave's latest issue of loads (made in M_jl) is in flight: exact
    // while that issue was a full one (K and V); near the end, where issues carry fewer loads,
    // wait for everything.  FULL: that issue was a full one.
    auto wait_older = [&]<bool FULL>(std::bool_constant<FULL>, int jl) CPATTN_AI {
        if (FULL || jl + 3 < nblk)
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * LOADS_PER_WAVE) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    if (first) {
        issue_prologue(cur);
        wait_prologue();
    }
    __syncthreads();      // every wave has waited for its own prologue loads

    // Both groups run M_0, SM_0, M_1, SM_1, ..., M_nblk; group 1 starts one slot late (an
    // extra barrier up front; group 0 adds one at the end), so on every SIMD one wave is in
    // an MFMA slot while the other is in a softmax slot.  A wave issues its pieces of
    // (K_{j+3}, V_{j+2}) inside its M_j slot, into the buffers of K_{j-1} and V_{j-2}, which
    // M_{j-1} of both groups finished reading before the previous barrier.  Before every
    // slot barrier a wave waits for all but its latest issue, so the blocks issued in M_{j-2}
    // are in LDS by the start of slot 2j+1: SM_j prefetches K_{j+1} fragments from there,
    // and M_{j+1} reads K_{j+1}, V_j.  The slot barrier itself does not wait for memory.
    auto slot_barrier = [&]() CPATTN_AI { asm volatile("s_barrier" ::: "memory"); };
    auto body = [&]<int R, bool QK, bool PV, bool USE_PRE, bool FULL = false>(
                    ic<R>, std::bool_constant<QK>, std::bool_constant<PV>, std::bool_constant<USE_PRE>, int j,
                    std::bool_constant<FULL> = {}) CPATTN_AI {
        M(ic<R>{}, std::bool_constant<QK>{}, std::bool_constant<PV>{}, std::bool_constant<USE_PRE>{},
          std::bool_constant<FULL>{}, j);
        __builtin_amdgcn_sched_barrier(0);
        wait_older(std::bool_constant<FULL>{}, j);
        __builtin_amdgcn_sched_barrier(0);
        slot_barrier();
        if constexpr (QK) {
            SM(ic<R>{}, std::bool_constant<FULL>{}, j);
            __builtin_amdgcn_sched_barrier(0);
            issue_part(ic<R>{}, ic<NP_M>{}, std::bool_constant<FULL>{}, j);
        }
        wait_older(std::bool_constant<FULL>{}, j);
        __builtin_amdgcn_sched_barrier(0);
        slot_barrier();
    };
    using T = std::true_type;
    using F = std::false_type;
    if (group != 0) slot_barrier();
    body(ic<0>{}, T{}, F{}, F{}, 0);
    int j = 1;
    // Steady state, with no runtime checks: every load these four blocks issue (K up to
    // block j+6, V up to j+5) is a full block, and none of them is the last block.  Each
    // check removed is a scalar branch in the MFMA or softmax stream; taken branches there
    // cost the schedule far more than their instructions (measured: 5% of the kernel).
    const int nfull = Skv / BN;
    for (; j + 7 <= nfull; j += 4) {
        body(ic<1>{}, T{}, T{}, T{}, j, T{});
        body(ic<2>{}, T{}, T{}, T{}, j + 1, T{});
        body(ic<3>{}, T{}, T{}, T{}, j + 2, T{});
        body(ic<0>{}, T{}, T{}, T{}, j + 3, T{});
    }
    // Dynamic schedule: claim the next unit now, a few blocks before the end, so that the
    // atomic's round trip overlaps the last blocks (it is complete by the end of the next
    // softmax slot, and its result is first read after the epilogue).
    unsigned long long claim = 0;
    if (map.sched != nullptr && tid == 0) claim = sched_ticket(map, k_unit, (int)blockIdx.x);
    for (; j + 3 < nblk; j += 4) {
        body(ic<1>{}, T{}, T{}, T{}, j);
        body(ic<2>{}, T{}, T{}, T{}, j + 1);
        body(ic<3>{}, T{}, T{}, T{}, j + 2);
        body(ic<0>{}, T{}, T{}, T{}, j + 3);
    }
    if (j < nblk) body(ic<1>{}, T{}, T{}, T{}, j);
    if (j + 1 < nblk) body(ic<2>{}, T{}, T{}, T{}, j + 1);
    if (j + 2 < nblk) body(ic<3>{}, T{}, T{}, T{}, j + 2);
    // The claimed unit goes to every wave through LDS; the barriers of the last body order it.
    if (map.sched != nullptr && tid == 0) {
        *next_lds = sched_next(map, k_unit, (int)blockIdx.x, (int)gridDim.x, claim);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    switch (nblk & 3) {      // M_nblk: the last PV product only
        case 0: body(ic<0>{}, F{}, T{}, F{}, nblk); break;
        case 1: body(ic<1>{}, F{}, T{}, F{}, nblk); break;
        case 2: body(ic<2>{}, F{}, T{}, F{}, nblk); break;
        default: body(ic<3>{}, F{}, T{}, F{}, nblk); break;
    }
    if (group == 0) slot_barrier();
    // No wave reads LDS from here on: the next unit's prologue goes out now, ahead of this unit's
    // epilogue (an accumulating epilogue first issues its own loads of the old O, so that its
    // wait does not also cover the prologue's).
    const int n_units = map.n_dp + map.n_split * map.split_s;
    // (read from LDS by every lane; readfirstlane tells the compiler the unit is wave-uniform, so
    // the branches on it below are scalar ones)
    const int next = map.sched != nullptr ? __builtin_amdgcn_readfirstlane(*next_lds) : static_next;
    const bool has_next = next >= 0 && next < n_units;

    // ---- epilogue: O = O / l, LSE = (m + log2 l) ln 2; a piece goes to the workspace, an
    // accumulating call folds the result into the (O, LSE) already in o/lse.
    // Accumulating rows load every old value they fold in first (the stores below go to the same
    // rows, so loads written after them could not move ahead of them and would each wait out a
    // round trip), then the next unit's prologue goes out (wave-uniform), then the arithmetic.
    // A lane whose row is past Sq works on row Sq - 1 (its Q, old O and LSE are that row's), so it
    // stores that row's own bits again: every wave issues the same stores on every path, which
    // lets the compiler's wait for the next prologue leave them all in flight.
    const bool acc_rows = OUT_F32 && map.accumulate && slot < 0;
    const int srow = min(qrow, Sq - 1);
    f32x4 old[OUT_F32 ? NDT * 4 : 1];
    float la = -INFINITY;
    if constexpr (OUT_F32) {
        if (acc_rows) {
            const int64_t orow = o_base + srow * o_row;
            la = lse[(size_t)bh * Sq + srow];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    old[dt * 4 + g] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + orow +
                                                                      dt * 32 + g * 8 + hh * 4);
            // In the tile that holds row Sq - 1, lanes of other waves also read that row (their rows
            // are past Sq) and write it back: every wave has its old values before any wave stores.
            if (cur.row0 + kBM > Sq) {
                asm volatile("" : "+v"(la));
#pragma unroll
                for (int i = 0; i < NDT * 4; ++i) asm volatile("" : "+v"(old[i]));
                __syncthreads();
            }
        }
    }
    if (has_next) issue_prologue(geom(next));
    const float l_tot = sum_across_halves(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_new = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    if (__builtin_amdgcn_readfirstlane(slot) >= 0) {      // wave-uniform: a scalar branch
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
        map.ws_lse[wrow] = lse_new;                // both lane halves hold the same value
        // The wait for the next prologue sits in each branch, in straight-line code after the Q
        // loads, so the compiler counts the stores between them; it is unconditional, so no path
        // back to the loop leaves qreg pending (without a next unit it returns at once).
        wait_prologue();
    } else {
        const int64_t orow = o_base + srow * o_row;
        float wa = 0.f, wb = inv, L = lse_new;   // O = wa * O_old + wb * acc
        if (acc_rows) {
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
        if constexpr (OUT_F32) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = dt * 32 + g * 8 + hh * 4;
                    f32x4 x = f32x4{oacc[dt][g * 4 + 0], oacc[dt][g * 4 + 1], oacc[dt][g * 4 + 2],
                                    oacc[dt][g * 4 + 3]} * wb;
                    if (acc_rows) x += old[dt * 4 + g] * wa;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow + d0) = x;
                }
        } else {
            // Lane half hh holds columns 8g + 4hh .. +3 of each 8-column group g.  For each pair of
            // groups (2p, 2p + 1) the halves swap one packed pair (v_permlane32_swap) so that half
            // hh holds all 8 columns of group 2p + hh and stores them as one 16-byte piece.
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    u32x2 pk[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int g = 2 * p + e;
                        const f32x4 x = f32x4{oacc[dt][g * 4 + 0], oacc[dt][g * 4 + 1], oacc[dt][g * 4 + 2],
                                              oacc[dt][g * 4 + 3]} * wb;
                        pk[e] = u32x2{pack16x2<F16>(x[0], x[1]), pack16x2<F16>(x[2], x[3])};
                    }
                    // low half: {own group 2p, the high half's group 2p}; high half: {the low half's
                    // group 2p + 1, own group 2p + 1}
                    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
                    const int d0 = dt * 32 + (2 * p + hh) * 8;
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(o) + orow + d0) =
                        u32x4{(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
                }
        }
        lse[(size_t)bh * Sq + srow] = L;           // both lane halves hold the same value
        wait_prologue();
    }
    return has_next ? next : -1;
}

// At most one workgroup per resident slot (gridDim.x of them, a multiple of the XCD count), each
// looping over work units, so a finished unit is followed by the next one without a new workgroup
// launch.  A unit's last LDS reads end before its final barrier, so the next unit's loads into the
// same buffers need no extra synchronisation.
//
// Static schedule (no counter): workgroup b runs b, b + gridDim.x, ... of a grid of units in which
// ids are dealt round-robin over the XCDs and mapped so that each XCD walks a contiguous range of
// whole tiles (then of pieces): the workgroups resident on one XCD share a head's K/V stream in
// its L2.
//
// Dynamic schedule (map.sched): per-XCD ranges of units with a shared tail (unit_sched.h).
template <int D, bool F16, bool OUT_F32, bool SEQ, bool KT>
__global__ __launch_bounds__(512) void attn_fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* __restrict__ o, float* __restrict__ lse, int Sq, int Skv_all, int nQt, int H, Strides sq, Strides skv,
    Strides so, AttnTileMap map, float c, int n_grid) {
    __shared__ int next_unit;
    const int n_units = map.n_dp + map.n_split * map.split_s;
    const bool dynamic = map.sched != nullptr;
    const int G = (int)gridDim.x;
    const int b = (int)blockIdx.x;
    int64_t bid = b;                       // static schedule: next grid id (64-bit: no overflow near INT_MAX)
    auto next_static = [&]() -> int {
        int u = -1;
        for (; bid < n_grid && u < 0; bid += G) u = sched_static_unit(map, bid);
        return u;
    };
    int u = dynamic ? sched_first(map, b) : next_static();
    u32x4 qreg[D / 16];                    // the current unit's Q^T operand (loaded by its prologue)
    bool first = true;
    while (u >= 0 && u < n_units) {       // one call site: the unit body is inlined once
        const int after = dynamic ? -1 : next_static();
        u = attn_unit<D, F16, OUT_F32, SEQ, KT>(u, first, after, qreg, q, k, v, o, lse, Sq, Skv_all, nQt, H, sq, skv,
                                            so, map, c, &next_unit);
        first = false;
    }
}

// Clears the dynamic schedule's counters (kSchedWords words) before a launch that uses one.
__global__ void zero_sched_kernel(unsigned long long* sched) {
    for (int i = threadIdx.x; i < kSchedWords; i += blockDim.x) sched[i] = 0;
}

template <int D, bool F16, bool OUT_F32, bool SEQ, bool KT>
hipError_t launch(const AttnFwdArgs& a) {
    const int nQt = (int)((a.Sq + kBM - 1) / kBM);
    const int64_t total = (int64_t)a.BH * nQt;
    const UnitGrid ug = sched_plan(total, a.split_tiles, a.split_pieces, a.slots, a.sched != nullptr);
    AttnTileMap m = ug.map;
    m.ws_o = a.ws_o;
    m.ws_lse = a.ws_lse;
    m.accumulate = a.accumulate ? 1 : 0;
    m.sched = a.sched;
    const int grid = ug.grid, launch_grid = ug.launch_grid;
    const float c = (float)((double)a.scale * 1.4426950408889634);
    if (a.sched != nullptr && a.sched_clear) {
        hipLaunchKernelGGL(zero_sched_kernel, dim3(1), dim3(256), 0, a.stream, a.sched_clear);
        const hipError_t ez = hipGetLastError();
        if (ez != hipSuccess) return ez;
    }
    hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, F16, OUT_F32, SEQ, KT>), dim3(launch_grid), dim3(512), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.o, a.lse, (int)a.Sq, (int)a.Skv, nQt, (int)a.H, a.sq,
                       a.skv, a.so, m, c, grid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_tiles == 0) return e;
    MergePiecesArgs f{a.ws_o, a.ws_lse, a.o, a.lse, m.n_dp, m.n_split, m.split_s, nQt, a.H, a.so, a.Sq, a.D,
                      a.out_f32 ? MergeOut::F32 : (F16 ? MergeOut::F16 : MergeOut::BF16), a.accumulate, a.stream};
    return launch_merge_pieces(f);
}

template <int D, bool F16, bool OUT_F32>
int occupancy() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_mfma_kernel<D, F16, OUT_F32, false, false>, 512, 0) !=
        hipSuccess)
        return 0;
    return n;
}

template <int D, bool F16, bool OUT_F32>
hipError_t launch_layout(const AttnFwdArgs& a) {
    return a.seq_major ? launch<D, F16, OUT_F32, true, false>(a) : launch<D, F16, OUT_F32, false, false>(a);
}

// Q, K, V and O head-major or sequence-major (the K-sequence-last layout has units of its own).
template <bool F16>
hipError_t launch_any(const AttnFwdArgs& a) {
    if (a.D == 128) return a.out_f32 ? launch_layout<128, F16, true>(a) : launch_layout<128, F16, false>(a);
    return a.out_f32 ? launch_layout<64, F16, true>(a) : launch_layout<64, F16, false>(a);
}

// K [B, H, D, Skv] (sequence last), Q, V and O head-major.
template <bool F16>
hipError_t launch_kt(const AttnFwdArgs& a) {
    if (a.D == 128)
        return a.out_f32 ? launch<128, F16, true, false, true>(a) : launch<128, F16, false, false, true>(a);
    return a.out_f32 ? launch<64, F16, true, false, true>(a) : launch<64, F16, false, false, true>(a);
}

}  // namespace
}  // namespace cpattn
