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
// Each row is handled inside one wave (lanes = 8-element chunks of the row),
// so an in-place call (o_out == o_a, lse_out == lse_a) is safe: every lane of
// the row loads both LSEs in the same instruction, before the one lane that
// writes lse_out, and each lane rewrites only the O chunk it read itself.
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

// Fast path (D/8 <= 64): each wave owns MU groups of 64/(D/8) rows; every lane loads all of
// its chunks (both operands, both LSEs) before computing and storing any of them.
template <MergeOut T, int MU>
__global__ __launch_bounds__(256) void attn_merge_kernel(const void* o_a, const float* lse_a, const void* o_b,
                                                         const float* lse_b, void* o_out, float* lse_out,
                                                         int64_t rows, int D, int rows_per_wave) {
    const int lane = threadIdx.x & 63;
    const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int tpr = D >> 3;
    const int r_in = lane / tpr;
    if (r_in >= rows_per_wave) return;
    const int ch = lane - r_in * tpr;
    constexpr bool F32 = T == MergeOut::F32;
    constexpr int NV = F32 ? 2 : 1;     // 16-byte vectors per 8-element chunk
    u32x4 a[MU][NV], b[MU][NV];
    float la[MU], lb[MU];
    int64_t row[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
        row[u] = (gwave * MU + u) * rows_per_wave + r_in;
        if (row[u] < rows) {
            la[u] = lse_a[row[u]];
            lb[u] = lse_b[row[u]];
            const size_t off = ((size_t)row[u] * D + (size_t)ch * 8) * (F32 ? 4 : 2) / 16;
#pragma unroll
            for (int w = 0; w < NV; ++w) {
                a[u][w] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_a) + off + w);
                b[u][w] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_b) + off + w);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
        if (row[u] >= rows) continue;
        float wa, wb, L;
        merge_weights(la[u], lb[u], wa, wb, L);
        const size_t off = ((size_t)row[u] * D + (size_t)ch * 8) * (F32 ? 4 : 2) / 16;
        if constexpr (F32) {
#pragma unroll
            for (int w = 0; w < NV; ++w) {
                const f32x4 x = __builtin_bit_cast(f32x4, a[u][w]), y = __builtin_bit_cast(f32x4, b[u][w]);
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x * wa + y * wb),
                                            reinterpret_cast<u32x4*>(o_out) + off + w);
            }
        } else {
            u32x4 r;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float alo = lo16<T>(a[u][0][w]), ahi = hi16<T>(a[u][0][w]);
                const float blo = lo16<T>(b[u][0][w]), bhi = hi16<T>(b[u][0][w]);
                r[w] = pack16<T>(__builtin_fmaf(alo, wa, blo * wb), __builtin_fmaf(ahi, wa, bhi * wb));
            }
            __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(o_out) + off);
        }
        if (ch == 0) lse_out[row[u]] = L;
    }
}

// General path (D/8 > 64): one row per wave, lanes loop over the row's chunks.
template <MergeOut T>
__global__ __launch_bounds__(256) void attn_merge_wide_kernel(const void* o_a, const float* lse_a, const void* o_b,
                                                              const float* lse_b, void* o_out, float* lse_out,
                                                              int64_t rows, int D) {
    const int lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (row >= rows) return;
    constexpr bool F32 = T == MergeOut::F32;
    float wa, wb, L;
    merge_weights(lse_a[row], lse_b[row], wa, wb, L);
    const int tpr = D >> 3;
    for (int ch = lane; ch < tpr; ch += 64) {
        const size_t off = (size_t)row * D + (size_t)ch * 8;
        if constexpr (F32) {
            const f32x4* pa = reinterpret_cast<const f32x4*>(static_cast<const float*>(o_a) + off);
            const f32x4* pb = reinterpret_cast<const f32x4*>(static_cast<const float*>(o_b) + off);
            const f32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
            f32x4* po = reinterpret_cast<f32x4*>(static_cast<float*>(o_out) + off);
            po[0] = a0 * wa + b0 * wb;
            po[1] = a1 * wa + b1 * wb;
        } else {
            const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o_a) + off);
            const u32x4 b = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o_b) + off);
            u32x4 r;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float alo = lo16<T>(a[w]), ahi = hi16<T>(a[w]);
                const float blo = lo16<T>(b[w]), bhi = hi16<T>(b[w]);
                r[w] = pack16<T>(__builtin_fmaf(alo, wa, blo * wb), __builtin_fmaf(ahi, wa, bhi * wb));
            }
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(o_out) + off) = r;
        }
    }
    if (lane == 0) lse_out[row] = L;
}

// Merge of the key-range pieces of split attention tiles.  The same fold over n
// partials: M = max_p L_p, L = M + ln sum_p e^(L_p - M), O = sum_p e^(L_p - L) O_p,
// where the partials are the tile's pieces (normalised f32 O, natural LSE) and,
// when accumulating, the (O, LSE) already in o/lse.  One row per D/4 lanes, four
// elements per lane.
template <MergeOut T>
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
    const float la = accumulate ? lse[row] : -INFINITY;
    float mx = la;
    for (int p = 0; p < pieces; ++p) mx = fmaxf(mx, lp[(size_t)p * TR]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = -INFINITY;
    if (mx != -INFINITY) {
        float tot = expf(la - mx);
        for (int p = 0; p < pieces; ++p) tot += expf(lp[(size_t)p * TR] - mx);
        L = mx + logf(tot);
        if (accumulate) acc = *reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + orow + c4) *
                              expf(la - L);
        for (int p = 0; p < pieces; ++p)
            acc += *reinterpret_cast<const f32x4*>(op + (size_t)p * TR * D) * expf(lp[(size_t)p * TR] - L);
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

template <MergeOut T>
hipError_t launch_merge_typed(const MergeArgs& a) {
    const int D = (int)a.D;
    const int tpr = D / 8;
    if (tpr > 64) {
        const int64_t blocks = (a.rows + 3) / 4;
        hipLaunchKernelGGL(attn_merge_wide_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, a.stream, a.o_a,
                           a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, D);
        return hipGetLastError();
    }
    constexpr int MU = 1;   // row groups per wave (measured best on MI355X)
    const int rpw = 64 / tpr;
    const int64_t waves = (a.rows + (int64_t)rpw * MU - 1) / ((int64_t)rpw * MU);
    const int64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((attn_merge_kernel<T, MU>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.o_a,
                       a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, D, rpw);
    return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeArgs& a) {
    switch (a.o_type) {
        case MergeOut::F32: return launch_merge_typed<MergeOut::F32>(a);
        case MergeOut::F16: return launch_merge_typed<MergeOut::F16>(a);
        default: return launch_merge_typed<MergeOut::BF16>(a);
    }
}

template <MergeOut T>
void launch_pieces_typed(const MergePiecesArgs& a, int64_t blocks) {
    hipLaunchKernelGGL(merge_pieces_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, a.stream, a.ws_o, a.ws_lse, a.o,
                       a.lse, a.first_tile, a.n_split, a.pieces, a.nQt, (int)a.H, a.so, a.Sq, (int)a.D,
                       a.accumulate ? 1 : 0);
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
