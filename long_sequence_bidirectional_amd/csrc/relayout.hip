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

// n / d for 32-bit n by a 64-bit multiply-high: m = ceil(2^64 / d) makes the quotient exact
// for every n < 2^32 (the rounding error of m is below d, so it shifts n * m / 2^64 by less
// than n / 2^64 < 1 / d).  d = 1 takes m = 0 and returns n.
struct FastDiv {
    uint32_t d;
    uint64_t m;
};
FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.m = d <= 1 ? 0 : (~0ull / d) + 1;
    return f;
}
__device__ __forceinline__ uint32_t div_of(uint32_t n, const FastDiv& f) {
    return f.d == 1 ? n : (uint32_t)__umul64hi(f.m, (uint64_t)n);
}

struct RelayoutDivs {
    FastDiv Hp, S_l, P, S, H, cpr;
};

__device__ __forceinline__ uint32_t src_row_of(uint32_t r, int mode, const RelayoutDivs& q) {
    if (mode == 0 || mode == 2) {
        const uint32_t t = div_of(r, q.Hp), h = r - t * q.Hp.d;
        const uint32_t t2 = div_of(t, q.S_l), s = t - t2 * q.S_l.d;
        const uint32_t b = div_of(t2, q.P), p = t2 - b * q.P.d;
        return mode == 0 ? (b * q.S_l.d + s) * q.H.d + p * q.Hp.d + h : (b * q.Hp.d + h) * q.S.d + p * q.S_l.d + s;
    }
    if (mode == 1) {
        const uint32_t t = div_of(r, q.S), ts = r - t * q.S.d;
        const uint32_t b = div_of(t, q.Hp), h = t - b * q.Hp.d;
        const uint32_t p = div_of(ts, q.S_l), s = ts - p * q.S_l.d;
        return ((b * q.P.d + p) * q.S_l.d + s) * q.Hp.d + h;
    }
    const uint32_t t = div_of(r, q.H), hg = r - t * q.H.d;
    const uint32_t b = div_of(t, q.S_l), s = t - b * q.S_l.d;
    const uint32_t g = div_of(hg, q.Hp), h = hg - g * q.Hp.d;
    return ((b * q.P.d + g) * q.S_l.d + s) * q.Hp.d + h;
}

// A workgroup moves tiles of whole rows (about kTileChunks 16-byte chunks each, contiguous in
// dst), visiting tiles with a grid stride; within a tile consecutive lanes take consecutive
// chunks (every access coalesced) and each thread issues its UNROLL loads before its stores.
// Measured on MI355X for three [5520, 24, 128] bf16 shards from HBM: 5.7 TB/s, against 5.1 TB/s
// for a plain device-to-device copy of the same bytes.
constexpr int kRelayoutThreads = 256;
constexpr int UNROLL = 2;
constexpr uint32_t kTileChunks = kRelayoutThreads * UNROLL;
// One launch moves up to kMaxRelayoutTensors tensors of the same shape (blockIdx.y picks the
// tensor), so the three tensors of one all-to-all share one launch's ramp and drain.
__global__ __launch_bounds__(kRelayoutThreads) void relayout_kernel(RelayoutPtrs ptrs, uint32_t n_rows,
                                                                    uint32_t tile_rows, uint64_t n_tiles, int mode,
                                                                    RelayoutDivs q) {
    const u32x4* __restrict__ src = static_cast<const u32x4*>(ptrs.src[blockIdx.y]);
    u32x4* __restrict__ dst = static_cast<u32x4*>(ptrs.dst[blockIdx.y]);
    const uint32_t cpr = q.cpr.d;
    const uint32_t tile_chunks = tile_rows * cpr;
    for (uint64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        const uint64_t r0 = tile * tile_rows;
        for (uint32_t l0 = threadIdx.x; l0 < tile_chunks; l0 += kTileChunks) {
            u32x4 val[UNROLL];
            uint64_t di[UNROLL];
            bool ok[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const uint32_t l = l0 + u * kRelayoutThreads;
                const uint32_t lr = div_of(l, q.cpr), c = l - lr * cpr;
                const uint64_t r = r0 + lr;
                ok[u] = l < tile_chunks && r < n_rows;
                di[u] = r * cpr + c;
                if (ok[u]) {
                    const uint32_t sr = src_row_of((uint32_t)r, mode, q);
                    val[u] = __builtin_nontemporal_load(&src[(uint64_t)sr * cpr + c]);
                }
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                if (ok[u]) __builtin_nontemporal_store(val[u], &dst[di[u]]);
        }
    }
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
    RelayoutDivs q;
    q.Hp = make_fastdiv(Hp);
    q.S_l = make_fastdiv((uint32_t)a.S_local);
    q.P = make_fastdiv((uint32_t)a.P);
    q.S = make_fastdiv((uint32_t)(a.P * a.S_local));
    q.H = make_fastdiv((uint32_t)a.H);
    q.cpr = make_fastdiv(cpr);
    const uint32_t tile_rows = cpr >= kTileChunks ? 1u : kTileChunks / cpr;
    const uint64_t n_tiles = ((uint64_t)n_rows + tile_rows - 1) / tile_rows;
    const uint64_t blocks = n_tiles < kMaxStrideBlocks ? n_tiles : kMaxStrideBlocks;
    hipLaunchKernelGGL(relayout_kernel, dim3((unsigned)blocks, (unsigned)a.n_tensors), dim3(kRelayoutThreads), 0,
                       a.stream, a.ptrs, n_rows, tile_rows, n_tiles, a.mode, q);
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
