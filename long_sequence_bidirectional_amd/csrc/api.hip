// C ABI of libcpattn: argument validation (host only, before any HIP call)
// and dispatch to the gfx950 kernels.  Semantics are documented in
// include/cpattn.h.
#include <math.h>

#include <initializer_list>
#include <stdint.h>

#include "../../include/cpattn.h"
#include "kernels.h"

#define CPATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 62;

// a * b, or -1 if either is negative or the product reaches kMaxElems.
int64_t mul_checked(int64_t a, int64_t b) {
    if (a < 0 || b < 0) return -1;
    if (a == 0 || b == 0) return 0;
    if (a > kMaxElems / b) return -1;
    return a * b;
}

int64_t prod(std::initializer_list<int64_t> xs) {
    int64_t p = 1;
    for (int64_t x : xs) {
        p = mul_checked(p, x);
        if (p < 0) return -1;
    }
    return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};
Range range(const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + (uintptr_t)bytes};
}
bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;   // empty ranges never overlap
    return a.lo < b.hi && b.lo < a.hi;
}

int64_t dtype_size(cpattn_dtype t) { return t == CPATTN_BF16 ? 2 : 4; }
bool dtype_valid(int t) { return t == CPATTN_BF16 || t == CPATTN_F32; }

bool dims_ok(std::initializer_list<int64_t> xs, int64_t min_value) {
    for (int64_t x : xs)
        if (x < min_value || x > kMaxDim) return false;
    return true;
}

cpattn_status hip_status(hipError_t e) { return e == hipSuccess ? CPATTN_OK : CPATTN_E_HIP; }

struct AttnCheck {
    int64_t q_elems, kv_elems, rows;
};

// Shared checks of attn_fwd and ring_attn_fwd (dtype pair already resolved).
cpattn_status check_attn_shapes(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                int64_t tile_rows, AttnCheck* out) {
    if (!dims_ok({B, H, Sq}, 1) || !dims_ok({Skv}, 0)) return CPATTN_E_SHAPE;
    if (D != 64 && D != 128) return CPATTN_E_HEADDIM;
    if (!(scale > 0.f) || !isfinite(scale)) return CPATTN_E_SCALE;
    const int64_t q_elems = prod({B, H, Sq, D});
    const int64_t kv_elems = prod({B, H, Skv, D});
    const int64_t rows = prod({B, H, Sq});
    if (q_elems < 0 || kv_elems < 0 || rows < 0) return CPATTN_E_SHAPE;
    // workgroup count must fit the kernels' 32-bit tile index
    const int64_t tiles = prod({B, H, (Sq + tile_rows - 1) / tile_rows});
    if (tiles < 0 || tiles + 8 > kMaxDim) return CPATTN_E_SHAPE;
    out->q_elems = q_elems;
    out->kv_elems = kv_elems;
    out->rows = rows;
    return CPATTN_OK;
}

cpattn_status run_attn(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t Sq,
                       int64_t Skv, int64_t D, float scale, cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                       hipStream_t stream) {
    if (Skv == 0)
        return hip_status(cpattn::launch_fill_empty(o, BH * Sq * D * dtype_size(o_dtype), lse, BH * Sq, stream));
    cpattn::AttnFwdArgs a{q, k, v, o, lse, BH, Sq, Skv, D, scale, o_dtype == CPATTN_F32, stream};
    return hip_status(in_dtype == CPATTN_BF16 ? cpattn::launch_attn_fwd_bf16(a) : cpattn::launch_attn_fwd_f32(a));
}

}  // namespace

CPATTN_EXPORT cpattn_status cpattn_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                            int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                            cpattn_dtype in_dtype, cpattn_dtype o_dtype, hipStream_t stream) {
    if (!q || !o || !lse || (Skv != 0 && (!k || !v))) return CPATTN_E_NULL;
    if (!dtype_valid(in_dtype) || !dtype_valid(o_dtype)) return CPATTN_E_DTYPE;
    if (in_dtype == CPATTN_F32 && o_dtype != CPATTN_F32) return CPATTN_E_DTYPE;
    AttnCheck c;
    const cpattn_status st = check_attn_shapes(B, H, Sq, Skv, D, scale, 32, &c);
    if (st != CPATTN_OK) return st;
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse) || (Skv && (!aligned16(k) || !aligned16(v))))
        return CPATTN_E_ALIGN;
    const int64_t isz = dtype_size(in_dtype), osz = dtype_size(o_dtype);
    const Range rq = range(q, c.q_elems * isz), rk = range(k, c.kv_elems * isz), rv = range(v, c.kv_elems * isz);
    const Range ro = range(o, c.q_elems * osz), rl = range(lse, c.rows * 4);
    if (overlap(ro, rl) || overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) ||
        overlap(rl, rk) || overlap(rl, rv))
        return CPATTN_E_ALIAS;
    return run_attn(q, k, v, o, lse, B * H, Sq, Skv, D, scale, in_dtype, o_dtype, stream);
}

CPATTN_EXPORT cpattn_status cpattn_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                                              const float* lse_b, void* o_out, float* lse_out, int64_t B,
                                              int64_t H, int64_t S, int64_t D, cpattn_dtype o_dtype,
                                              hipStream_t stream) {
    if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return CPATTN_E_NULL;
    if (!dtype_valid(o_dtype)) return CPATTN_E_DTYPE;
    if (!dims_ok({B, H, S}, 1)) return CPATTN_E_SHAPE;
    const int64_t osz = dtype_size(o_dtype);
    if (D < 8 || D > 1024 || (D * osz) % 16 != 0) return CPATTN_E_HEADDIM;
    const int64_t rows = prod({B, H, S});
    const int64_t elems = prod({B, H, S, D});
    if (rows < 0 || elems < 0 || rows > (kMaxDim - 1) * 4) return CPATTN_E_SHAPE;
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out) || !aligned16(lse_a) || !aligned16(lse_b) ||
        !aligned16(lse_out))
        return CPATTN_E_ALIGN;
    const Range ra = range(o_a, elems * osz), rb = range(o_b, elems * osz), ro = range(o_out, elems * osz);
    const Range la = range(lse_a, rows * 4), lb = range(lse_b, rows * 4), lo = range(lse_out, rows * 4);
    // o_out: exactly o_a, exactly o_b, or disjoint from both; same for lse_out.
    if ((o_out != o_a && overlap(ro, ra)) || (o_out != o_b && overlap(ro, rb))) return CPATTN_E_ALIAS;
    if ((lse_out != lse_a && overlap(lo, la)) || (lse_out != lse_b && overlap(lo, lb))) return CPATTN_E_ALIAS;
    if (overlap(ro, la) || overlap(ro, lb) || overlap(ro, lo) || overlap(lo, ra) || overlap(lo, rb))
        return CPATTN_E_ALIAS;
    cpattn::MergeArgs m{o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, D, o_dtype == CPATTN_F32, stream};
    return hip_status(cpattn::launch_attn_merge(m));
}

CPATTN_EXPORT cpattn_status cpattn_ring_attn_fwd(const void* q, const void* k_chunks, const void* v_chunks,
                                                 float* o, float* lse, float* o_work, float* lse_work, int64_t B,
                                                 int64_t H, int64_t Sq, int64_t Skv_chunk, int64_t n_chunks,
                                                 int64_t D, float scale, hipStream_t stream) {
    if (!q || !o || !lse) return CPATTN_E_NULL;
    if (n_chunks < 1 || n_chunks > kMaxDim) return CPATTN_E_SHAPE;
    if (Skv_chunk != 0 && (!k_chunks || !v_chunks)) return CPATTN_E_NULL;
    if (n_chunks > 1 && (!o_work || !lse_work)) return CPATTN_E_NULL;
    AttnCheck c;
    const cpattn_status st = check_attn_shapes(B, H, Sq, Skv_chunk, D, scale, 32, &c);
    if (st != CPATTN_OK) return st;
    const int64_t all_kv = mul_checked(c.kv_elems, n_chunks);
    if (all_kv < 0) return CPATTN_E_SHAPE;
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse) ||
        (Skv_chunk && (!aligned16(k_chunks) || !aligned16(v_chunks))) ||
        (n_chunks > 1 && (!aligned16(o_work) || !aligned16(lse_work))))
        return CPATTN_E_ALIGN;
    const Range rq = range(q, c.q_elems * 2), rk = range(k_chunks, all_kv * 2), rv = range(v_chunks, all_kv * 2);
    const Range ro = range(o, c.q_elems * 4), rl = range(lse, c.rows * 4);
    const Range rw = n_chunks > 1 ? range(o_work, c.q_elems * 4) : Range{0, 0};
    const Range rlw = n_chunks > 1 ? range(lse_work, c.rows * 4) : Range{0, 0};
    const Range outs[4] = {ro, rl, rw, rlw};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], rq) || overlap(outs[i], rk) || overlap(outs[i], rv)) return CPATTN_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return CPATTN_E_ALIAS;
    }
    const int64_t BH = B * H;
    const int64_t chunk_bytes = c.kv_elems * 2;
    cpattn_status s = run_attn(q, k_chunks, v_chunks, o, lse, BH, Sq, Skv_chunk, D, scale, CPATTN_BF16,
                               CPATTN_F32, stream);
    for (int64_t ch = 1; ch < n_chunks && s == CPATTN_OK; ++ch) {
        const char* kc = static_cast<const char*>(k_chunks) + ch * chunk_bytes;
        const char* vc = static_cast<const char*>(v_chunks) + ch * chunk_bytes;
        s = run_attn(q, kc, vc, o_work, lse_work, BH, Sq, Skv_chunk, D, scale, CPATTN_BF16, CPATTN_F32, stream);
        if (s != CPATTN_OK) break;
        cpattn::MergeArgs m{o, lse, o_work, lse_work, o, lse, c.rows, D, true, stream};
        s = hip_status(cpattn::launch_attn_merge(m));
    }
    return s;
}

namespace {

cpattn_status relayout(const void* src, void* dst, int64_t B, int64_t S_local, int64_t H, int64_t D, int64_t P,
                       cpattn_dtype dt, cpattn_dir dir, bool pack, hipStream_t stream) {
    if (!src || !dst) return CPATTN_E_NULL;
    if (!dtype_valid(dt)) return CPATTN_E_DTYPE;
    if (dir != CPATTN_SEQ_TO_HEAD && dir != CPATTN_HEAD_TO_SEQ) return CPATTN_E_SHAPE;
    if (!dims_ok({B, S_local, H, D, P}, 1) || H % P != 0) return CPATTN_E_SHAPE;
    const int64_t row_bytes = D * dtype_size(dt);
    if (row_bytes % 16 != 0) return CPATTN_E_HEADDIM;
    const int64_t n_rows = prod({B, S_local, H});
    const int64_t bytes = mul_checked(n_rows, row_bytes);
    // 32-bit row indices in the kernel; one thread per 16-byte chunk.
    if (n_rows < 0 || bytes < 0 || n_rows > (int64_t)UINT32_MAX || bytes / 16 / 256 >= kMaxDim)
        return CPATTN_E_SHAPE;
    if (!aligned16(src) || !aligned16(dst)) return CPATTN_E_ALIGN;
    if (overlap(range(src, bytes), range(dst, bytes))) return CPATTN_E_ALIAS;
    const int mode = (dir == CPATTN_SEQ_TO_HEAD ? 0 : 2) + (pack ? 0 : 1);
    cpattn::RelayoutArgs a{src, dst, B, S_local, H, P, row_bytes, mode, stream};
    return hip_status(cpattn::launch_relayout(a));
}

}  // namespace

CPATTN_EXPORT cpattn_status cpattn_ulysses_pack(const void* src, void* dst, int64_t B, int64_t S_local, int64_t H,
                                                int64_t D, int64_t P, cpattn_dtype dt, cpattn_dir dir,
                                                hipStream_t stream) {
    return relayout(src, dst, B, S_local, H, D, P, dt, dir, true, stream);
}

CPATTN_EXPORT cpattn_status cpattn_ulysses_unpack(const void* src, void* dst, int64_t B, int64_t S_local,
                                                  int64_t H, int64_t D, int64_t P, cpattn_dtype dt,
                                                  cpattn_dir dir, hipStream_t stream) {
    return relayout(src, dst, B, S_local, H, D, P, dt, dir, false, stream);
}

CPATTN_EXPORT const char* cpattn_status_string(cpattn_status s) {
    switch (s) {
        case CPATTN_OK: return "ok";
        case CPATTN_E_NULL: return "a required pointer is NULL";
        case CPATTN_E_SHAPE: return "a size is out of range, inconsistent or overflows";
        case CPATTN_E_DTYPE: return "unsupported dtype or dtype combination";
        case CPATTN_E_HEADDIM: return "head dimension not supported";
        case CPATTN_E_ALIGN: return "a pointer is not 16-byte aligned";
        case CPATTN_E_ALIAS: return "buffers overlap where overlap is not allowed";
        case CPATTN_E_HIP: return "the HIP runtime rejected a launch";
        case CPATTN_E_SCALE: return "the score scale is not a finite positive number";
    }
    return "unknown status";
}

CPATTN_EXPORT int cpattn_abi_version(void) { return CPATTN_ABI_VERSION; }
