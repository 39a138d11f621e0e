// Merge of two partial attention results (O, LSE) over disjoint key sets.
//
// Ring Attention keeps an online softmax while K/V chunks stream past the
// local queries ("Scaling AI inference across multiple GPUs using NVIDIA
// TensorRT with multi-device inference support", section "Ring Attention");
// each chunk's partial result folds into the running one by
//   M = max(La, Lb),  L = M + ln(e^(La-M) + e^(Lb-M)),  O = e^(La-L) Oa + e^(Lb-L) Ob.
// An empty side (LSE = -inf) contributes weight 0; two empty sides give
// O = 0, LSE = -inf.
//
// HBM-bound: per row it reads 2*D values of O and two LSEs and writes D + 1.
// A row of O is D*sizeof(O)/16 16-byte vectors (the entry point requires a
// whole number of them).  Each row is handled inside one wave, one vector per
// lane, so an in-place call (o_out == o_a, lse_out == lse_a) is safe: every
// lane of the row loads both LSEs in the same instruction, before the one lane
// that writes lse_out, and each lane rewrites only the vectors it read itself.
#include "common.h"
#include "kernels.h"

namespace cpattn {
namespace {

// Widen the low / high 16-bit halves of a packed pair of the 16-bit O type.
template <MergeOut T>
__device__ __forceinline__ float lo16(uint32_t w) {
    if constexpr (T == MergeOut::F16) return f16_bits_to_f32(w & 0xFFFFu);
    else return __uint_as_float(w << 16);
}
template <MergeOut T>
__device__ __forceinline__ float hi16(uint32_t w) {
    if constexpr (T == MergeOut::F16) return f16_bits_to_f32(w >> 16);
    else return __uint_as_float(w & 0xFFFF0000u);
}
template <MergeOut T>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
    if constexpr (T == MergeOut::F16) return pack_f16x2(lo, hi);
    else return pack_bf16x2(lo, hi);
}

__device__ __forceinline__ void merge_weights(float la, float lb, float& wa, float& wb, float& L) {
    const float m = fmaxf(la, lb);
    wa = 0.f;
    wb = 0.f;
    L = -INFINITY;
    if (m != -INFINITY) {
        const float ea = expf(la - m);
        const float eb = expf(lb - m);
        const float tot = ea + eb;
        L = m + logf(tot);
        wa = ea / tot;
        wb = eb / tot;
    }
}

// One 16-byte vector of a row: 4 f32 or 8 16-bit values of O.
template <MergeOut T>
__device__ __forceinline__ u32x4 merge_vec(const u32x4& a, const u32x4& b, float wa, float wb) {
    if constexpr (T == MergeOut::F32) {
        const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
        return __builtin_bit_cast(u32x4, x * wa + y * wb);
    } else {
        u32x4 r;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            r[w] = pack16<T>(__builtin_fmaf(lo16<T>(a[w]), wa, lo16<T>(b[w]) * wb),
                             __builtin_fmaf(hi16<T>(a[w]), wa, hi16<T>(b[w]) * wb));
        return r;
    }
}

// Fast path (a row of vr <= 64 16-byte vectors): a wave owns MU groups of rpw = 64 / vr
// consecutive rows, one vector per lane and group, so each load or store instruction covers
// rpw whole rows of O contiguously.  Every lane loads all of its vectors (both operands, both
// LSEs) before computing and storing any of them.
template <MergeOut T, int MU>
__global__ __launch_bounds__(256) void attn_merge_kernel(const void* o_a, const float* lse_a, const void* o_b,
                                                         const float* lse_b, void* o_out, float* lse_out,
                                                         int64_t rows, int vr, int rpw) {
    const int lane = threadIdx.x & 63;
    const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int r_in = lane / vr;
    if (r_in >= rpw) return;
    const int vec = lane - r_in * vr;
    const u32x4* pa = static_cast<const u32x4*>(o_a);
    const u32x4* pb = static_cast<const u32x4*>(o_b);
    u32x4 a[MU], b[MU];
    float la[MU], lb[MU];
    int64_t row[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
        row[u] = (gwave * MU + u) * rpw + r_in;
        if (row[u] < rows) {
            la[u] = lse_a[row[u]];
            lb[u] = lse_b[row[u]];
            const size_t off = (size_t)row[u] * vr + vec;
            a[u] = __builtin_nontemporal_load(pa + off);
            b[u] = __builtin_nontemporal_load(pb + off);
        }
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
        if (row[u] >= rows) continue;
        float wa, wb, L;
        merge_weights(la[u], lb[u], wa, wb, L);
        __builtin_nontemporal_store(merge_vec<T>(a[u], b[u], wa, wb),
                                    static_cast<u32x4*>(o_out) + (size_t)row[u] * vr + vec);
        if (vec == 0) lse_out[row[u]] = L;
    }
}

// General path (vr > 64): one row per wave, lanes loop over the row's vectors, two at a time.
template <MergeOut T>
__global__ __launch_bounds__(256) void attn_merge_wide_kernel(const void* o_a, const float* lse_a, const void* o_b,
                                                              const float* lse_b, void* o_out, float* lse_out,
                                                              int64_t rows, int vr) {
    const int lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (row >= rows) return;
    float wa, wb, L;
    merge_weights(lse_a[row], lse_b[row], wa, wb, L);
    const u32x4* pa = static_cast<const u32x4*>(o_a) + (size_t)row * vr;
    const u32x4* pb = static_cast<const u32x4*>(o_b) + (size_t)row * vr;
    u32x4* po = static_cast<u32x4*>(o_out) + (size_t)row * vr;
    int v = lane;
    for (; v + 64 < vr; v += 128) {
        const u32x4 a0 = pa[v], a1 = pa[v + 64], b0 = pb[v], b1 = pb[v + 64];
        po[v] = merge_vec<T>(a0, b0, wa, wb);
        po[v + 64] = merge_vec<T>(a1, b1, wa, wb);
    }
    if (v < vr) po[v] = merge_vec<T>(pa[v], pb[v], wa, wb);
    if (lane == 0) lse_out[row] = L;
}

// Merge of the key-range pieces of split attention tiles.  The same fold over n
// partials: M = max_p L_p, L = M + ln sum_p e^(L_p - M), O = sum_p e^(L_p - L) O_p,
// where the partials are the tile's pieces (normalised f32 O, natural LSE) and,
// when accumulating, the (O, LSE) already in o/lse.  One row per D/4 lanes, four
// elements per lane.
// NP > 0: at most NP pieces, all read in one batch (the host picks the smallest instantiated NP
// that holds the tile's pieces); NP = 0: any count, read in batches.
template <MergeOut T, int NP>
__global__ __launch_bounds__(256) void merge_pieces_kernel(const float* __restrict__ ws_o,
                                                           const float* __restrict__ ws_lse, void* o, float* lse,
                                                           int first_tile, int n_split, int pieces, int nQt, int H,
                                                           Strides so, int64_t Sq, int D, int accumulate) {
    constexpr int TR = kAttnTileRows;
    const int lpr = D >> 2;                       // lanes per row
    const int64_t grow = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / lpr;
    const int c4 = ((int)threadIdx.x % lpr) * 4;
    const int ti = (int)(grow / TR);
    const int r = (int)(grow - (int64_t)ti * TR);
    if (ti >= n_split) return;
    const int tile = first_tile + ti;
    const int bh = tile / nQt;
    const int64_t qrow = (int64_t)(tile - bh * nQt) * TR + r;
    if (qrow >= Sq) return;
    const size_t row = (size_t)bh * Sq + qrow;                                  // lse index
    const int64_t orow = (bh / H) * so.batch + (bh % H) * so.head + qrow * so.row;   // o offset
    const float* lp = ws_lse + (size_t)ti * pieces * TR + r;
    const float* op = ws_o + ((size_t)ti * pieces * TR + r) * D + c4;
    // With NP > 0 every piece's LSE and O and the old row are read in one batch of independent
    // loads (indices clamped to the last piece, values past it ignored), so the merge costs one
    // memory round trip; otherwise the pieces are read in batches.  Both paths fold in the same
    // order, so they give the same bits.
    const float la = accumulate ? lse[row] : -INFINITY;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = -INFINITY;
    if constexpr (NP > 0) {
        float l[NP];
        f32x4 ov[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const size_t pc = (size_t)min(i, pieces - 1);
            l[i] = lp[pc * TR];
            ov[i] = *reinterpret_cast<const f32x4*>(op + pc * TR * D);
        }
        const f32x4 old = accumulate ? *reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + orow + c4)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
        float mx = la;
#pragma unroll
        for (int i = 0; i < NP; ++i)
            if (i < pieces) mx = fmaxf(mx, l[i]);
        if (mx != -INFINITY) {
            float tot = expf(la - mx);
#pragma unroll
            for (int i = 0; i < NP; ++i)
                if (i < pieces) tot += expf(l[i] - mx);
            L = mx + logf(tot);
            if (accumulate) acc = old * expf(la - L);
#pragma unroll
            for (int i = 0; i < NP; ++i)
                if (i < pieces) acc += ov[i] * expf(l[i] - L);
        }
    } else {
        constexpr int LB = 16, OB = 8;
        float mx = la;
        for (int p0 = 0; p0 < pieces; p0 += LB) {
            float l[LB];
#pragma unroll
            for (int i = 0; i < LB; ++i) l[i] = lp[(size_t)min(p0 + i, pieces - 1) * TR];
#pragma unroll
            for (int i = 0; i < LB; ++i)
                if (p0 + i < pieces) mx = fmaxf(mx, l[i]);
        }
        if (mx != -INFINITY) {
            float tot = expf(la - mx);
            for (int p0 = 0; p0 < pieces; p0 += LB) {
                float l[LB];
#pragma unroll
                for (int i = 0; i < LB; ++i) l[i] = lp[(size_t)min(p0 + i, pieces - 1) * TR];
#pragma unroll
                for (int i = 0; i < LB; ++i)
                    if (p0 + i < pieces) tot += expf(l[i] - mx);
            }
            L = mx + logf(tot);
            if (accumulate) acc = *reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + orow + c4) *
                                  expf(la - L);
            for (int p0 = 0; p0 < pieces; p0 += OB) {
                f32x4 ov[OB];
                float l[OB];
#pragma unroll
                for (int i = 0; i < OB; ++i) {
                    const size_t pc = (size_t)min(p0 + i, pieces - 1);
                    ov[i] = *reinterpret_cast<const f32x4*>(op + pc * TR * D);
                    l[i] = lp[pc * TR];
                }
#pragma unroll
                for (int i = 0; i < OB; ++i)
                    if (p0 + i < pieces) acc += ov[i] * expf(l[i] - L);
            }
        }
    }
    if constexpr (T == MergeOut::F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow + c4) = acc;
    } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + orow + c4) =
            u32x2{pack16<T>(acc[0], acc[1]), pack16<T>(acc[2], acc[3])};
    }
    if (c4 == 0) lse[row] = L;
}

}  // namespace

// Row groups per wave of the fast path.  Measured on MI355X, f32 O [1,24,5520,128] in place:
// 32.8 us with one, 33.2 with two, 38.8 with four (and 38.3 before the vector layout, whose f32
// loads and stores each covered every other 16 bytes of a row).  16-bit O: 18.2 us with one, two
// or four.
constexpr int kMergeMU = 1;

int64_t attn_merge_blocks(int64_t rows, int64_t D, MergeOut t) {
    const int64_t vr = D * (t == MergeOut::F32 ? 4 : 2) / 16;   // 16-byte vectors per row
    if (vr > 64) return (rows + 3) / 4;                         // one row per wave
    const int64_t per_wave = (64 / vr) * kMergeMU;
    return ((rows + per_wave - 1) / per_wave + 3) / 4;
}

template <MergeOut T>
hipError_t launch_merge_typed(const MergeArgs& a) {
    constexpr int osz = T == MergeOut::F32 ? 4 : 2;
    const int vr = (int)(a.D * osz / 16);   // 16-byte vectors per row (the entry point checks divisibility)
    const int64_t blocks = attn_merge_blocks(a.rows, a.D, T);   // the entry point keeps blocks * 256 < 2^32
    if (vr > 64) {
        hipLaunchKernelGGL(attn_merge_wide_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, a.stream, a.o_a,
                           a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, vr);
        return hipGetLastError();
    }
    const int rpw = 64 / vr;
    hipLaunchKernelGGL((attn_merge_kernel<T, kMergeMU>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.o_a,
                       a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, vr, rpw);
    return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeArgs& a) {
    switch (a.o_type) {
        case MergeOut::F32: return launch_merge_typed<MergeOut::F32>(a);
        case MergeOut::F16: return launch_merge_typed<MergeOut::F16>(a);
        default: return launch_merge_typed<MergeOut::BF16>(a);
    }
}

template <MergeOut T, int NP>
void launch_pieces_np(const MergePiecesArgs& a, int64_t blocks) {
    hipLaunchKernelGGL((merge_pieces_kernel<T, NP>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.ws_o, a.ws_lse,
                       a.o, a.lse, a.first_tile, a.n_split, a.pieces, a.nQt, (int)a.H, a.so, a.Sq, (int)a.D,
                       a.accumulate ? 1 : 0);
}

// Piece counts read in one batch: the smallest of these that holds a tile's pieces (the planner's
// usual counts lie between 4 and 36; more pieces take the batched path).
template <MergeOut T>
void launch_pieces_typed(const MergePiecesArgs& a, int64_t blocks) {
    if (a.pieces <= 4) launch_pieces_np<T, 4>(a, blocks);
    else if (a.pieces <= 8) launch_pieces_np<T, 8>(a, blocks);
    else if (a.pieces <= 12) launch_pieces_np<T, 12>(a, blocks);
    else if (a.pieces <= 16) launch_pieces_np<T, 16>(a, blocks);
    else if (a.pieces <= 24) launch_pieces_np<T, 24>(a, blocks);
    else if (a.pieces <= 36) launch_pieces_np<T, 36>(a, blocks);
    else launch_pieces_np<T, 0>(a, blocks);
}

hipError_t launch_merge_pieces(const MergePiecesArgs& a) {
    const int lpr = (int)(a.D / 4);
    const int64_t threads = (int64_t)a.n_split * kAttnTileRows * lpr;
    const int64_t blocks = (threads + 255) / 256;
    switch (a.out) {
        case MergeOut::F32: launch_pieces_typed<MergeOut::F32>(a, blocks); break;
        case MergeOut::F16: launch_pieces_typed<MergeOut::F16>(a, blocks); break;
        default: launch_pieces_typed<MergeOut::BF16>(a, blocks); break;
    }
    return hipGetLastError();
}

}  // namespace cpattn
