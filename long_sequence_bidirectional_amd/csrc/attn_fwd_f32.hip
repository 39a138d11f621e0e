// Non-causal attention forward, all-f32 path (plain FMA, no matrix cores).
//
// Same online-softmax recurrence as the bf16 kernel (K/V streamed in blocks,
// running max and sum per query row; "Scaling AI inference across multiple
// GPUs using NVIDIA TensorRT with multi-device inference support", section
// "Ring Attention"), with every product, sum and the output kept in f32.
//
// Work split: a workgroup of 256 threads owns 32 query rows of one (b, h);
// 8 consecutive lanes share a row, lane `sub` holding dims 4*sub + 32*i ..+3
// of q and of the output accumulator.  K and V blocks of 32 keys are staged
// in LDS; each score is a per-lane partial dot product reduced over the 8
// lanes of the row.
#include "common.h"
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int FBM = 32;   // query rows per workgroup
constexpr int FBN = 32;   // keys per block

__device__ __forceinline__ float sum8(float x) {
    x += __shfl_xor(x, 1, 8);
    x += __shfl_xor(x, 2, 8);
    x += __shfl_xor(x, 4, 8);
    return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                           const float* __restrict__ v, float* __restrict__ o,
                                                           float* __restrict__ lse, int Sq, int Skv, int nQt,
                                                           int H, Strides sq, Strides skv, Strides so, float c) {
    constexpr int NI = D / 32;   // float4 groups per lane
    __shared__ __attribute__((aligned(16))) float Kf[FBN * D];
    __shared__ __attribute__((aligned(16))) float Vf[FBN * D];

    const int bh = blockIdx.x / nQt;
    const int qt = blockIdx.x - bh * nQt;
    const int tid = threadIdx.x;
    const int r = tid >> 3;
    const int sub = tid & 7;
    const int qrow = qt * FBM + r;
    const int b = bh / H, h = bh - (bh / H) * H;
    const float* qp = q + b * sq.batch + h * sq.head;
    const float* kp = k + b * skv.batch + h * skv.head;
    const float* vp = v + b * skv.batch + h * skv.head;

    f32x4 qv[NI], ov[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        qv[i] = qrow < Sq ? *reinterpret_cast<const f32x4*>(qp + qrow * sq.row + sub * 4 + 32 * i)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        ov[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m_run = -INFINITY, l_run = 0.f;

    const int nblk = (Skv + FBN - 1) / FBN;
    for (int j = 0; j < nblk; ++j) {
        __syncthreads();
        for (int e = tid; e < FBN * D / 4; e += 256) {
            const int row = e / (D / 4);
            const int col = e - row * (D / 4);
            const int key = j * FBN + row;
            f32x4 kv4 = {0.f, 0.f, 0.f, 0.f}, vv4 = {0.f, 0.f, 0.f, 0.f};
            if (key < Skv) {
                kv4 = reinterpret_cast<const f32x4*>(kp + key * skv.row)[col];
                vv4 = reinterpret_cast<const f32x4*>(vp + key * skv.row)[col];
            }
            reinterpret_cast<f32x4*>(Kf)[e] = kv4;
            reinterpret_cast<f32x4*>(Vf)[e] = vv4;
        }
        __syncthreads();

        float s[FBN];
#pragma unroll
        for (int jj = 0; jj < FBN; ++jj) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const f32x4 kk = *reinterpret_cast<const f32x4*>(&Kf[jj * D + sub * 4 + 32 * i]);
                part = __builtin_fmaf(qv[i][0], kk[0], part);
                part = __builtin_fmaf(qv[i][1], kk[1], part);
                part = __builtin_fmaf(qv[i][2], kk[2], part);
                part = __builtin_fmaf(qv[i][3], kk[3], part);
            }
            s[jj] = sum8(part);
            if (j * FBN + jj >= Skv) s[jj] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int jj = 1; jj < FBN; ++jj) mx = fmaxf(mx, s[jj]);
        const float m_new = fmaxf(m_run, mx * c);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) ov[i] *= alpha;
#pragma unroll
        for (int jj = 0; jj < FBN; ++jj) {
            const float p = exp2_fast(__builtin_fmaf(s[jj], c, -m_new));
            psum += p;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const f32x4 vv = *reinterpret_cast<const f32x4*>(&Vf[jj * D + sub * 4 + 32 * i]);
                ov[i][0] = __builtin_fmaf(p, vv[0], ov[i][0]);
                ov[i][1] = __builtin_fmaf(p, vv[1], ov[i][1]);
                ov[i][2] = __builtin_fmaf(p, vv[2], ov[i][2]);
                ov[i][3] = __builtin_fmaf(p, vv[3], ov[i][3]);
            }
        }
        l_run = l_run * alpha + psum;
    }

    if (qrow < Sq) {
        const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
        float* orow = o + b * so.batch + h * so.head + qrow * so.row;
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<f32x4*>(orow + sub * 4 + 32 * i) = ov[i] * inv;
        if (sub == 0) lse[(size_t)bh * Sq + qrow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a) {
    const int nQt = (int)((a.Sq + FBM - 1) / FBM);
    const int64_t grid = a.BH * nQt;
    const float c = (float)((double)a.scale * 1.4426950408889634);
    if (a.D == 128)
        hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, a.stream,
                           static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                           static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, (int)a.Sq,
                           (int)a.Skv, nQt, (int)a.H, a.sq, a.skv, a.so, c);
    else
        hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, a.stream,
                           static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                           static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, (int)a.Sq,
                           (int)a.Skv, nQt, (int)a.H, a.sq, a.skv, a.so, c);
    return hipGetLastError();
}

}  // namespace cpattn
