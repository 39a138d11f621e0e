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

template <bool F32>
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
template <bool F32, int MU>
__global__ __launch_bounds__(256) void attn_merge_kernel(const void* o_a, const float* lse_a, const void* o_b,
                                                         const float* lse_b, void* o_out, float* lse_out,
                                                         int64_t rows, int D, int rows_per_wave) {
    const int lane = threadIdx.x & 63;
    const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int tpr = D >> 3;
    const int r_in = lane / tpr;
    if (r_in >= rows_per_wave) return;
    const int ch = lane - r_in * tpr;
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
        merge_weights<F32>(la[u], lb[u], wa, wb, L);
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
                const float alo = __uint_as_float(a[u][0][w] << 16), ahi = __uint_as_float(a[u][0][w] & 0xFFFF0000u);
                const float blo = __uint_as_float(b[u][0][w] << 16), bhi = __uint_as_float(b[u][0][w] & 0xFFFF0000u);
                r[w] = pack_bf16x2(__builtin_fmaf(alo, wa, blo * wb), __builtin_fmaf(ahi, wa, bhi * wb));
            }
            __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(o_out) + off);
        }
        if (ch == 0) lse_out[row[u]] = L;
    }
}

// General path (D/8 > 64): one row per wave, lanes loop over the row's chunks.
template <bool F32>
__global__ __launch_bounds__(256) void attn_merge_wide_kernel(const void* o_a, const float* lse_a, const void* o_b,
                                                              const float* lse_b, void* o_out, float* lse_out,
                                                              int64_t rows, int D) {
    const int lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (row >= rows) return;
    float wa, wb, L;
    merge_weights<F32>(lse_a[row], lse_b[row], wa, wb, L);
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
                const float alo = __uint_as_float(a[w] << 16), ahi = __uint_as_float(a[w] & 0xFFFF0000u);
                const float blo = __uint_as_float(b[w] << 16), bhi = __uint_as_float(b[w] & 0xFFFF0000u);
                r[w] = pack_bf16x2(__builtin_fmaf(alo, wa, blo * wb), __builtin_fmaf(ahi, wa, bhi * wb));
            }
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(o_out) + off) = r;
        }
    }
    if (lane == 0) lse_out[row] = L;
}

}  // namespace

hipError_t launch_attn_merge(const MergeArgs& a) {
    const int D = (int)a.D;
    const int tpr = D / 8;
    if (tpr > 64) {
        const int64_t blocks = (a.rows + 3) / 4;
        if (a.f32)
            hipLaunchKernelGGL(attn_merge_wide_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, a.stream, a.o_a,
                               a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, D);
        else
            hipLaunchKernelGGL(attn_merge_wide_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                               a.o_a, a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, D);
        return hipGetLastError();
    }
    constexpr int MU = 1;   // row groups per wave (measured best on MI355X)
    const int rpw = 64 / tpr;
    const int64_t waves = (a.rows + (int64_t)rpw * MU - 1) / ((int64_t)rpw * MU);
    const int64_t blocks = (waves + 3) / 4;
    if (a.f32)
        hipLaunchKernelGGL((attn_merge_kernel<true, MU>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.o_a,
                           a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, D, rpw);
    else
        hipLaunchKernelGGL((attn_merge_kernel<false, MU>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.o_a,
                           a.lse_a, a.o_b, a.lse_b, a.o_out, a.lse_out, a.rows, D, rpw);
    return hipGetLastError();
}

}  // namespace cpattn
