// Ulysses sequence<->head relayout (pack before / unpack after each all-to-all).
//
// DeepSpeed Ulysses swaps a sequence split for a head split with one
// all-to-all before attention and swaps back with a second one after it
// ("Scaling AI inference across multiple GPUs using NVIDIA TensorRT with
// multi-device inference support", section "DeepSpeed Ulysses").  Around each
// exchange a rank reorders whole D-vectors ("rows") between its token-major
// shard, the [P, S_local, Hp] send/receive buffer and the head-major
// full-sequence layout that attention reads.  The four maps (row indices,
// Hp = H / P):
//   mode 0  pack   seq->head  dst[b,p,s,h]        <- src[b,s,p*Hp+h]
//   mode 1  unpack seq->head  dst[b,h,p*S_l+s]    <- src[b,p,s,h]
//   mode 2  pack   head->seq  dst[b,p,s,h]        <- src[b,h,p*S_l+s]
//   mode 3  unpack head->seq  dst[b,s,g*Hp+h]     <- src[b,g,s,h]
//
// A pure copy, so HBM-bound: every byte is read once and written once.  The
// kernel walks dst in order; each row is a contiguous run of row_bytes (a
// multiple of 16) in both buffers, moved with 16-byte loads and stores by
// consecutive lanes.  The source row index is derived once per row.
#include "common.h"
#include "kernels.h"

namespace cpattn {
namespace {

// Source row of destination row r (the divisors are uniform, so the compiler computes each
// reciprocal once per thread).
__device__ __forceinline__ uint32_t src_row_of(uint32_t r, int mode, uint32_t S_l, uint32_t H, uint32_t Hp,
                                               uint32_t P) {
    if (mode == 0 || mode == 2) {
        const uint32_t h = r % Hp;
        uint32_t t = r / Hp;
        const uint32_t s = t % S_l;
        t /= S_l;
        const uint32_t p = t % P;
        const uint32_t b = t / P;
        return mode == 0 ? (b * S_l + s) * H + p * Hp + h : (b * Hp + h) * (P * S_l) + p * S_l + s;
    }
    if (mode == 1) {
        const uint32_t S = P * S_l;
        const uint32_t ts = r % S;
        const uint32_t t = r / S;
        const uint32_t h = t % Hp;
        const uint32_t b = t / Hp;
        const uint32_t p = ts / S_l;
        const uint32_t s = ts - p * S_l;
        return ((b * P + p) * S_l + s) * Hp + h;
    }
    const uint32_t hg = r % H;
    const uint32_t t = r / H;
    const uint32_t s = t % S_l;
    const uint32_t b = t / S_l;
    const uint32_t g = hg / Hp;
    const uint32_t h = hg - g * Hp;
    return ((b * P + g) * S_l + s) * Hp + h;
}

// Each thread moves UNROLL 16-byte chunks spaced one grid-width apart (consecutive lanes take
// consecutive chunks of dst, so every access is coalesced); all loads are issued before the
// first store to keep enough bytes in flight for HBM.  Measured on MI355X against one contiguous
// tile of rows per workgroup and against division by multiply-high: this form is the fastest
// of the three for [5520, 24, 128] bf16 shards from HBM.
constexpr int kRelayoutThreads = 256;
constexpr int UNROLL = 2;   // chunks in flight per thread (measured best among 1, 2, 4 and 8)
__device__ __forceinline__ void relayout_body(const u32x4* __restrict__ src, u32x4* __restrict__ dst, uint32_t n_rows,
                                              uint32_t cpr, int mode, uint32_t S_l, uint32_t H, uint32_t Hp,
                                              uint32_t P) {
    const uint64_t total = (uint64_t)n_rows * cpr;
    const uint64_t stride = (uint64_t)gridDim.x * kRelayoutThreads;
    const bool small = total <= (uint64_t)UINT32_MAX;     // chunk ids fit a 32-bit division
    for (uint64_t id = (uint64_t)blockIdx.x * kRelayoutThreads + threadIdx.x; id < total; id += stride * UNROLL) {
        u32x4 val[UNROLL];
        uint64_t di[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint64_t cid = id + (uint64_t)u * stride;
            di[u] = cid;
            if (cid < total) {
                const uint32_t r = small ? (uint32_t)cid / cpr : (uint32_t)(cid / cpr);
                const uint32_t c = (uint32_t)(cid - (uint64_t)r * cpr);
                const uint32_t sr = src_row_of(r, mode, S_l, H, Hp, P);
                val[u] = __builtin_nontemporal_load(&src[(uint64_t)sr * cpr + c]);
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            if (di[u] < total) __builtin_nontemporal_store(val[u], &dst[di[u]]);
    }
}

__global__ __launch_bounds__(kRelayoutThreads) void relayout_kernel(const u32x4* __restrict__ src,
                                                                    u32x4* __restrict__ dst, uint32_t n_rows,
                                                                    uint32_t cpr, int mode, uint32_t S_l, uint32_t H,
                                                                    uint32_t Hp, uint32_t P) {
    relayout_body(src, dst, n_rows, cpr, mode, S_l, H, Hp, P);
}

// Several tensors of one shape in one launch (blockIdx.y picks the tensor), so the three tensors
// of one all-to-all share one launch's ramp and drain.  A separate kernel: the pointer table costs
// each workgroup one more dependent scalar load at its start, which the single-tensor calls skip.
__global__ __launch_bounds__(kRelayoutThreads) void relayout_multi_kernel(RelayoutPtrs ptrs, uint32_t n_rows,
                                                                          uint32_t cpr, int mode, uint32_t S_l,
                                                                          uint32_t H, uint32_t Hp, uint32_t P) {
    relayout_body(static_cast<const u32x4*>(ptrs.src[blockIdx.y]), static_cast<u32x4*>(ptrs.dst[blockIdx.y]), n_rows,
                  cpr, mode, S_l, H, Hp, P);
}

__global__ __launch_bounds__(256) void fill_empty_kernel(u32x4* __restrict__ o, uint64_t o_chunks,
                                                         float* __restrict__ lse, uint64_t n_rows) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < o_chunks || gid < n_rows;
         gid += stride) {
        if (gid < o_chunks) o[gid] = u32x4{0, 0, 0, 0};
        if (gid < n_rows) lse[gid] = -INFINITY;
    }
}

// Both kernels above walk their range with a grid stride, so a launch is capped at this many
// workgroups (2^30 work-items, inside the 2^32 a launch may hold) and any size still fits.
constexpr uint64_t kMaxStrideBlocks = uint64_t(1) << 22;

}  // namespace

hipError_t launch_relayout(const RelayoutArgs& a) {
    const uint32_t Hp = (uint32_t)(a.H / a.P);
    const uint32_t cpr = (uint32_t)(a.row_bytes / 16);
    const uint32_t n_rows = (uint32_t)(a.B * a.S_local * a.H);
    const uint64_t total = (uint64_t)n_rows * cpr;
    uint64_t blocks = (total + kRelayoutThreads * UNROLL - 1) / (kRelayoutThreads * UNROLL);
    if (blocks > kMaxStrideBlocks) blocks = kMaxStrideBlocks;
    if (a.n_tensors == 1)
        hipLaunchKernelGGL(relayout_kernel, dim3((unsigned)blocks), dim3(kRelayoutThreads), 0, a.stream,
                           static_cast<const u32x4*>(a.ptrs.src[0]), static_cast<u32x4*>(a.ptrs.dst[0]), n_rows, cpr,
                           a.mode, (uint32_t)a.S_local, (uint32_t)a.H, Hp, (uint32_t)a.P);
    else
        hipLaunchKernelGGL(relayout_multi_kernel, dim3((unsigned)blocks, (unsigned)a.n_tensors),
                           dim3(kRelayoutThreads), 0, a.stream, a.ptrs, n_rows, cpr, a.mode, (uint32_t)a.S_local,
                           (uint32_t)a.H, Hp, (uint32_t)a.P);
    return hipGetLastError();
}

hipError_t launch_fill_empty(void* o, int64_t o_bytes, float* lse, int64_t n_rows, hipStream_t stream) {
    const uint64_t chunks = (uint64_t)o_bytes / 16;
    const uint64_t n = chunks > (uint64_t)n_rows ? chunks : (uint64_t)n_rows;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > kMaxStrideBlocks) blocks = kMaxStrideBlocks;
    hipLaunchKernelGGL(fill_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<u32x4*>(o),
                       chunks, lse, (uint64_t)n_rows);
    return hipGetLastError();
}

}  // namespace cpattn
