// QK-RMSNorm prologue of the attention sample.
//
// Before scaled dot-product attention, Q and K each go through an RMSNorm over
// head_dim evaluated in fp32 -- y = x * rsqrt(mean(x^2) + eps) * w -- and are
// cast back to the 16-bit model type; then each is multiplied by the fourth
// root of 1/head_dim, the score scale split over Q and K ("TensorRT
// multi-device attention inference in practice", step 1).  Here the scale is
// an optional 16-bit constant applied to the 16-bit RMSNorm output; the
// product of two 16-bit values is exact in f32, so it is rounded once.
//
// HBM-bound: every row of D 16-bit values is read once and written once.  A
// row lives in D/8 consecutive lanes of one wave (8 elements, 16 bytes per
// lane), so an in-place call is safe: the lanes of a row load it in one
// instruction before any of them stores.
#include "common.h"
#include "kernels.h"

namespace cpattn {
namespace {

template <bool F16>
__device__ __forceinline__ float widen(uint32_t w, int half) {
    const uint32_t b = half ? (w >> 16) : (w & 0xFFFFu);
    return F16 ? f16_bits_to_f32(b) : __uint_as_float(b << 16);
}

template <bool F16>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi) {
    return F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

template <bool F16>
__global__ __launch_bounds__(256) void qk_rmsnorm_kernel(const u32x4* x, const u32x4* __restrict__ w, u32x4* y,
                                                         int64_t rows, int lpr, float inv_d, float eps,
                                                         float scale16, int has_scale) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid / lpr;
    const int c = (int)(gid - row * lpr);      // this lane's 16-byte chunk of the row
    const bool valid = row < rows;
    const u32x4 xv = valid ? x[row * lpr + c] : u32x4{0u, 0u, 0u, 0u};
    const u32x4 wv = w[c];
    float xf[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        xf[e] = widen<F16>(xv[e >> 1], e & 1);
        ss = __builtin_fmaf(xf[e], xf[e], ss);
    }
    for (int m = 1; m < lpr; m <<= 1) ss += __shfl_xor(ss, m, lpr);
    const float r = 1.0f / sqrtf(ss * inv_d + eps);
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) v[h] = xf[2 * p + h] * r * widen<F16>(wv[p], h);
        uint32_t q = narrow2<F16>(v[0], v[1]);          // the cast back to the 16-bit type
        if (has_scale) q = narrow2<F16>(widen<F16>(q, 0) * scale16, widen<F16>(q, 1) * scale16);
        out[p] = q;
    }
    if (valid) y[row * lpr + c] = out;
}

}  // namespace

hipError_t launch_qk_rmsnorm(const QkNormArgs& a) {
    const int lpr = (int)(a.D / 8);
    const int64_t threads = a.rows * lpr;
    const int64_t blocks = (threads + 255) / 256;
    const float inv_d = 1.0f / (float)a.D;
    if (a.f16)
        hipLaunchKernelGGL(qk_rmsnorm_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                           static_cast<const u32x4*>(a.x), static_cast<const u32x4*>(a.w), static_cast<u32x4*>(a.y),
                           a.rows, lpr, inv_d, a.eps, a.scale16, a.has_scale ? 1 : 0);
    else
        hipLaunchKernelGGL(qk_rmsnorm_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                           static_cast<const u32x4*>(a.x), static_cast<const u32x4*>(a.w), static_cast<u32x4*>(a.y),
                           a.rows, lpr, inv_d, a.eps, a.scale16, a.has_scale ? 1 : 0);
    return hipGetLastError();
}

}  // namespace cpattn
