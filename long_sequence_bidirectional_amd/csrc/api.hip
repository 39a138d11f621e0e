// C ABI of libcpattn: argument validation (host only, before any HIP call)
// and dispatch to the gfx950 kernels.  Semantics are documented in
// include/cpattn.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <initializer_list>
#include <stdint.h>

#include "../../include/cpattn.h"
#include "kernels.h"

#define CPATTN_EXPORT extern "C" __attribute__((visibility("default")))

static_assert(cpattn::kSchedBytes == CPATTN_WORKSPACE_COUNTER_BYTES, "workspace counter area");

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

// A C caller may pass any int in an enum argument, while in C++ a value outside the
// enumerators' bit range is not a valid value of the enum type.  Entry points therefore
// read each enum argument's bits as an int, validate that, and only then convert back.
template <class E>
int enum_bits(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

int64_t dtype_size(int t) { return t == CPATTN_F32 ? 4 : 2; }
bool dtype_valid(int t) { return t == CPATTN_BF16 || t == CPATTN_F32 || t == CPATTN_F16; }
bool dtype_16bit(int t) { return t == CPATTN_BF16 || t == CPATTN_F16; }

cpattn::MergeOut merge_out(int t) {
    return t == CPATTN_F32 ? cpattn::MergeOut::F32 : t == CPATTN_F16 ? cpattn::MergeOut::F16 : cpattn::MergeOut::BF16;
}

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

// ---- key-range split of the last, partial wave of tiles
//
// The bf16 kernel runs one tile (kAttnTileRows query rows of one (b, h)) per
// workgroup, and `slots` workgroups are resident at once.  With T tiles the last
// wave holds only T mod slots of them; splitting each of those tiles' keys into s
// pieces gives the tail ceil(rem * s / slots) rounds of 1/s tile plus a fixed
// cost per piece, which the planner minimises over s.
// A piece has at least 8 key blocks: its fixed cost (Q load, pipeline fill, epilogue) is then at
// most about half its work, and the dynamic schedule lets the workgroups of faster XCDs start the
// tail's pieces early, so fewer, longer pieces finish no later (ring chunk 5520 x 5520: 10 pieces
// of 8-9 blocks per split tile run 1.9% faster than 16 of 5-6).
constexpr int64_t kMinPieceBlocks = 8;      // key blocks (64 keys) per piece, at least
constexpr double kPieceCostBlocks = 4.0;    // fixed cost of a piece, in key blocks
constexpr int64_t kMaxPieces = 64;          // pieces per tile, at most

struct SplitPlan {
    int64_t tiles = 0, split_tiles = 0, pieces = 1;
    uint64_t bytes = 0;   // workspace used
};

uint64_t piece_bytes(int64_t D) { return (uint64_t)cpattn::kAttnTileRows * (uint64_t)(D + 1) * 4u; }

SplitPlan plan_split(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, int64_t slots, uint64_t ws_bytes) {
    SplitPlan p;
    p.tiles = BH * ((Sq + cpattn::kAttnTileRows - 1) / cpattn::kAttnTileRows);
    const int64_t nblk = (Skv + 63) / 64;
    if (slots <= 0 || nblk < 2 * kMinPieceBlocks) return p;
    const int64_t rem = p.tiles % slots;
    if (rem == 0) return p;
    const uint64_t max_pieces_ws = ws_bytes / piece_bytes(D);
    const int64_t s_max = std::min<int64_t>(kMaxPieces, nblk / kMinPieceBlocks);
    double best = 1.0;   // the unsplit tail: one round of whole tiles
    int64_t best_s = 1;
    for (int64_t s = 2; s <= s_max; ++s) {
        if ((uint64_t)(rem * s) > max_pieces_ws) break;
        const int64_t rounds = (rem * s + slots - 1) / slots;
        const double cost = (double)rounds * (1.0 / (double)s + kPieceCostBlocks / (double)nblk);
        if (cost < best - 1e-9) {
            best = cost;
            best_s = s;
        }
    }
    if (best_s == 1) return p;
    p.split_tiles = rem;
    p.pieces = best_s;
    p.bytes = (uint64_t)(rem * best_s) * piece_bytes(D);
    return p;
}

// Workgroups of an attention kernel resident at once on the current device (0 if unknown),
// cached per device, kernel (16-bit D = 64, D = 128, fp8) and output type.
int64_t device_slots(int64_t D, bool out_f32, bool fp8 = false) {
    constexpr int kCachedDevices = 64;
    static std::atomic<int64_t> cache[kCachedDevices][3][2];
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const int kind = fp8 ? 2 : (D == 128 ? 1 : 0);
    std::atomic<int64_t>* slot = (dev >= 0 && dev < kCachedDevices) ? &cache[dev][kind][out_f32 ? 1 : 0] : nullptr;
    if (slot) {
        const int64_t v = slot->load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const int64_t v = (int64_t)cus * (fp8 ? cpattn::attn_fwd_fp8_blocks_per_cu(out_f32)
                                          : cpattn::attn_fwd_bf16_blocks_per_cu(D, out_f32));
    if (slot && v > 0) slot->store(v, std::memory_order_relaxed);
    return v;
}

// Strides of an attention operand with S rows per (b, h) in the given layout.
cpattn::Strides layout_strides(int64_t H, int64_t S, int64_t D, bool seq_major) {
    if (seq_major) return cpattn::Strides{S * H * D, D, H * D};
    return cpattn::Strides{H * S * D, S * D, D};
}

// Attention of one K/V set into (o, lse): written, or folded into them when accumulate.
// ws_o/ws_lse (capacity ws_pieces pieces each) hold the partials of a split; null = no split.
// sched (a set of cpattn::kSchedSetWords words of device memory) enables the dynamic unit
// schedule; null = static.  When sched_clear is not null, the cpattn::kSchedWords words there
// (sched among them) are cleared first; when it is null, sched must already be zero.
cpattn_status run_attn(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                       int64_t Sq, int64_t Skv, int64_t D, float scale, cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                       bool accumulate, bool seq_major, float* ws_o, float* ws_lse, int64_t ws_pieces,
                       unsigned long long* sched, unsigned long long* sched_clear, hipStream_t stream,
                       bool k_seq_last = false) {
    const int64_t BH = B * H;
    if (Skv == 0) {   // empty key set: O = 0, LSE = -inf, the identity of the fold
        if (accumulate) return CPATTN_OK;
        return hip_status(cpattn::launch_fill_empty(o, BH * Sq * D * dtype_size(o_dtype), lse, BH * Sq, stream));
    }
    cpattn::AttnFwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.BH = BH;
    a.H = H;
    a.seq_major = seq_major;
    a.k_seq_last = k_seq_last;
    a.sq = layout_strides(H, Sq, D, seq_major);
    a.skv = layout_strides(H, Skv, D, seq_major);
    a.so = a.sq;
    a.Sq = Sq;
    a.Skv = Skv;
    a.D = D;
    a.scale = scale;
    a.out_f32 = o_dtype == CPATTN_F32;
    a.accumulate = accumulate;
    a.split_tiles = 0;
    a.split_pieces = 1;
    a.slots = 0;
    a.sched = nullptr;
    a.sched_clear = nullptr;
    a.stream = stream;
    if (in_dtype == CPATTN_F32) return hip_status(cpattn::launch_attn_fwd_f32(a));
    a.sched = sched;
    a.sched_clear = sched ? sched_clear : nullptr;
    a.slots = device_slots(D, a.out_f32);
    if (ws_o && ws_lse && ws_pieces > 0) {
        const SplitPlan p = plan_split(BH, Sq, Skv, D, a.slots, (uint64_t)ws_pieces * piece_bytes(D));
        if (p.split_tiles > 0) {
            a.split_tiles = p.split_tiles;
            a.split_pieces = p.pieces;
            a.ws_o = ws_o;
            a.ws_lse = ws_lse;
        }
    }
    if (k_seq_last)
        return hip_status(in_dtype == CPATTN_F16 ? cpattn::launch_attn_fwd_f16_kt(a)
                                                 : cpattn::launch_attn_fwd_bf16_kt(a));
    return hip_status(in_dtype == CPATTN_F16 ? cpattn::launch_attn_fwd_f16(a) : cpattn::launch_attn_fwd_bf16(a));
}

struct AttnFwdCheck {
    AttnCheck c;
    Range rq, rk, rv, ro, rl;
};

// Checks shared by attn_fwd and attn_fwd_ex (everything but the workspace).
cpattn_status check_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                             int64_t Sq, int64_t Skv, int64_t D, float scale, int in_dtype, int o_dtype,
                             AttnFwdCheck* out) {
    if (!q || !o || !lse || (Skv != 0 && (!k || !v))) return CPATTN_E_NULL;
    if (!dtype_valid(in_dtype) || !dtype_valid(o_dtype)) return CPATTN_E_DTYPE;
    if (o_dtype != in_dtype && o_dtype != CPATTN_F32) return CPATTN_E_DTYPE;   // O in the input type or f32
    AttnCheck& c = out->c;
    const cpattn_status st = check_attn_shapes(B, H, Sq, Skv, D, scale, 32, &c);
    if (st != CPATTN_OK) return st;
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse) || (Skv && (!aligned16(k) || !aligned16(v))))
        return CPATTN_E_ALIGN;
    const int64_t isz = dtype_size(in_dtype), osz = dtype_size(o_dtype);
    out->rq = range(q, c.q_elems * isz);
    out->rk = range(k, c.kv_elems * isz);
    out->rv = range(v, c.kv_elems * isz);
    out->ro = range(o, c.q_elems * osz);
    out->rl = range(lse, c.rows * 4);
    const Range &rq = out->rq, &rk = out->rk, &rv = out->rv, &ro = out->ro, &rl = out->rl;
    if (overlap(ro, rl) || overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) ||
        overlap(rl, rk) || overlap(rl, rv))
        return CPATTN_E_ALIAS;
    return CPATTN_OK;
}

}  // namespace

CPATTN_EXPORT cpattn_status cpattn_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                            int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                            cpattn_dtype in_dtype, cpattn_dtype o_dtype, hipStream_t stream) {
    const int idt = enum_bits(in_dtype), odt = enum_bits(o_dtype);
    AttnFwdCheck ck;
    const cpattn_status st = check_attn_fwd(q, k, v, o, lse, B, H, Sq, Skv, D, scale, idt, odt, &ck);
    if (st != CPATTN_OK) return st;
    return run_attn(q, k, v, o, lse, B, H, Sq, Skv, D, scale, static_cast<cpattn_dtype>(idt),
                    static_cast<cpattn_dtype>(odt), false, false, nullptr, nullptr, 0, nullptr, nullptr, stream);
}

namespace {

// Checks of attn_fwd_ex other than those of its workspace (flags, tensors, dtypes, layout limits).
cpattn_status check_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale, int idt, int odt,
                                uint32_t flags, AttnFwdCheck* ck) {
    if ((flags & ~(uint32_t)(CPATTN_FLAG_ACCUMULATE | CPATTN_FLAG_SEQ_MAJOR | CPATTN_FLAG_K_SEQ_LAST)) != 0)
        return CPATTN_E_FLAGS;
    const bool acc = (flags & CPATTN_FLAG_ACCUMULATE) != 0;
    const bool seq_major = (flags & CPATTN_FLAG_SEQ_MAJOR) != 0;
    const bool k_last = (flags & CPATTN_FLAG_K_SEQ_LAST) != 0;
    if (seq_major && k_last) return CPATTN_E_FLAGS;
    const cpattn_status st = check_attn_fwd(q, k, v, o, lse, B, H, Sq, Skv, D, scale, idt, odt, ck);
    if (st != CPATTN_OK) return st;
    if (acc && (!dtype_16bit(idt) || odt != CPATTN_F32)) return CPATTN_E_DTYPE;
    // the 16-bit kernels address a 64-row K/V block with 32-bit byte offsets
    if (seq_major && H * D >= (int64_t(1) << 25)) return CPATTN_E_SHAPE;
    if (k_last) {
        if (!dtype_16bit(idt)) return CPATTN_E_DTYPE;
        // K rows of Skv keys, read in 16-byte chunks of 8 keys from offsets below 2^32 bytes
        if (Skv % 8 != 0 || D * Skv * 2 >= (int64_t(1) << 32)) return CPATTN_E_SHAPE;
    }
    return CPATTN_OK;
}

// attn_fwd_ex after every check, with a workspace of workspace_bytes at `workspace` (or none).
cpattn_status run_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                              int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale, int idt, int odt,
                              uint32_t flags, void* workspace, uint64_t workspace_bytes, hipStream_t stream) {
    int64_t ws_pieces = 0;
    float *ws_o = nullptr, *ws_lse = nullptr;
    unsigned long long* sched = nullptr;
    if (workspace && workspace_bytes >= (uint64_t)cpattn::kSchedBytes) {
        // layout: schedule counters [kSchedBytes], ws_o [pieces, tile rows, D], ws_lse [pieces, tile rows]
        sched = static_cast<unsigned long long*>(workspace);
        ws_pieces = (int64_t)((workspace_bytes - cpattn::kSchedBytes) / piece_bytes(D));
        ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + cpattn::kSchedBytes);
        ws_lse = ws_o + (size_t)ws_pieces * cpattn::kAttnTileRows * D;
    }
    return run_attn(q, k, v, o, lse, B, H, Sq, Skv, D, scale, static_cast<cpattn_dtype>(idt),
                    static_cast<cpattn_dtype>(odt), (flags & CPATTN_FLAG_ACCUMULATE) != 0,
                    (flags & CPATTN_FLAG_SEQ_MAJOR) != 0, ws_o, ws_lse, ws_pieces, sched, sched, stream,
                    (flags & CPATTN_FLAG_K_SEQ_LAST) != 0);
}

}  // namespace

CPATTN_EXPORT cpattn_status cpattn_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                                               int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                               float scale, cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                                               uint32_t flags, void* workspace, uint64_t workspace_bytes,
                                               hipStream_t stream) {
    const int idt = enum_bits(in_dtype), odt = enum_bits(o_dtype);
    AttnFwdCheck ck;
    const cpattn_status st = check_attn_fwd_ex(q, k, v, o, lse, B, H, Sq, Skv, D, scale, idt, odt, flags, &ck);
    if (st != CPATTN_OK) return st;
    if (workspace_bytes != 0 && !workspace) return CPATTN_E_NULL;
    if (workspace && workspace_bytes > 0) {
        if (!aligned16(workspace)) return CPATTN_E_ALIGN;
        if (workspace_bytes > (uint64_t)kMaxElems) return CPATTN_E_SHAPE;
        const Range rw = range(workspace, (int64_t)workspace_bytes);
        if (overlap(rw, ck.rq) || overlap(rw, ck.rk) || overlap(rw, ck.rv) || overlap(rw, ck.ro) ||
            overlap(rw, ck.rl))
            return CPATTN_E_ALIAS;
    }
    return run_attn_fwd_ex(q, k, v, o, lse, B, H, Sq, Skv, D, scale, idt, odt, flags, workspace, workspace_bytes,
                           stream);
}

// ---- the library's static scratch (cpattn_attn_fwd_ex_static)
//
// A file-scope device array: every device the library runs on holds its own copy, at its own
// address, from the first use on that device until the process ends.  In host code the name is
// only a handle for hipGetSymbolAddress, never an address: the device address is looked up once
// per device, with that device current, and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[CPATTN_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device (null if HIP cannot give it), kept per device.
void* static_scratch_ptr() {
    constexpr int kCachedDevices = 64;
    static std::atomic<void*> cache[kCachedDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::atomic<void*>* slot = (dev >= 0 && dev < kCachedDevices) ? &cache[dev] : nullptr;
    if (slot) {
        void* p = slot->load(std::memory_order_acquire);
        if (p) return p;
    }
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    if (slot) slot->store(ptr, std::memory_order_release);
    return ptr;
}

}  // namespace

CPATTN_EXPORT cpattn_status cpattn_attn_fwd_ex_static(const void* q, const void* k, const void* v, void* o,
                                                      float* lse, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                                      int64_t D, float scale, cpattn_dtype in_dtype,
                                                      cpattn_dtype o_dtype, uint32_t flags, uint64_t scratch_bytes,
                                                      hipStream_t stream) {
    const int idt = enum_bits(in_dtype), odt = enum_bits(o_dtype);
    AttnFwdCheck ck;
    const cpattn_status st = check_attn_fwd_ex(q, k, v, o, lse, B, H, Sq, Skv, D, scale, idt, odt, flags, &ck);
    if (st != CPATTN_OK) return st;
    if (scratch_bytes > (uint64_t)CPATTN_STATIC_SCRATCH_BYTES) return CPATTN_E_SHAPE;
    void* ws = nullptr;
    if (scratch_bytes > 0) {
        ws = static_scratch_ptr();
        if (!ws) return CPATTN_E_HIP;
    }
    return run_attn_fwd_ex(q, k, v, o, lse, B, H, Sq, Skv, D, scale, idt, odt, flags, ws, scratch_bytes, stream);
}

CPATTN_EXPORT cpattn_status cpattn_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                                int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                                float scale, float q_scale, float k_scale, float v_scale,
                                                cpattn_dtype o_dtype, uint32_t flags, void* workspace,
                                                uint64_t workspace_bytes, hipStream_t stream) {
    if ((flags & ~(uint32_t)(CPATTN_FLAG_SEQ_MAJOR | CPATTN_FLAG_ACCUMULATE)) != 0) return CPATTN_E_FLAGS;
    const bool seq_major = (flags & CPATTN_FLAG_SEQ_MAJOR) != 0;
    const bool acc = (flags & CPATTN_FLAG_ACCUMULATE) != 0;
    if (!q || !o || !lse || (Skv != 0 && (!k || !v))) return CPATTN_E_NULL;
    const int odt = enum_bits(o_dtype);
    if (odt != CPATTN_BF16 && odt != CPATTN_F32) return CPATTN_E_DTYPE;
    if (acc && odt != CPATTN_F32) return CPATTN_E_DTYPE;
    AttnCheck c;
    cpattn_status st = check_attn_shapes(B, H, Sq, Skv, D, scale, 32, &c);
    if (st != CPATTN_OK) return st;
    if (D != 128) return CPATTN_E_HEADDIM;
    if (seq_major && H * D >= (int64_t(1) << 25)) return CPATTN_E_SHAPE;   // 32-bit block offsets
    for (float s : {q_scale, k_scale, v_scale})
        if (!(s > 0.f) || !isfinite(s)) return CPATTN_E_SCALE;
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse) || (Skv && (!aligned16(k) || !aligned16(v))))
        return CPATTN_E_ALIGN;
    const int64_t osz = dtype_size(odt);
    const Range rq = range(q, c.q_elems), rk = range(k, c.kv_elems), rv = range(v, c.kv_elems);
    const Range ro = range(o, c.q_elems * osz), rl = range(lse, c.rows * 4);
    if (overlap(ro, rl) || overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) ||
        overlap(rl, rk) || overlap(rl, rv))
        return CPATTN_E_ALIAS;
    if (workspace_bytes != 0 && !workspace) return CPATTN_E_NULL;
    if (workspace && workspace_bytes > 0) {
        if (!aligned16(workspace)) return CPATTN_E_ALIGN;
        if (workspace_bytes > (uint64_t)kMaxElems) return CPATTN_E_SHAPE;
        const Range rw = range(workspace, (int64_t)workspace_bytes);
        if (overlap(rw, rq) || overlap(rw, rk) || overlap(rw, rv) || overlap(rw, ro) || overlap(rw, rl))
            return CPATTN_E_ALIAS;
    }
    if (Skv == 0) {   // empty key set: O = 0, LSE = -inf, the identity of the fold
        if (acc) return CPATTN_OK;
        return hip_status(cpattn::launch_fill_empty(o, c.q_elems * osz, lse, c.rows, stream));
    }
    cpattn::AttnFp8Args a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.BH = B * H;
    a.H = H;
    a.Sq = Sq;
    a.Skv = Skv;
    a.seq_major = seq_major;
    a.sq = layout_strides(H, Sq, D, seq_major);
    a.skv = layout_strides(H, Skv, D, seq_major);
    a.so = a.sq;
    a.scale = scale;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.out_f32 = odt == CPATTN_F32;
    a.accumulate = acc;
    a.split_tiles = 0;
    a.split_pieces = 1;
    a.slots = device_slots(D, a.out_f32, true);
    a.sched = nullptr;
    a.sched_clear = nullptr;
    a.stream = stream;
    if (workspace && workspace_bytes >= (uint64_t)cpattn::kSchedBytes) {
        // same layout as attn_fwd_ex: counters, then the pieces' O, then their LSE
        a.sched = static_cast<unsigned long long*>(workspace);
        a.sched_clear = a.sched;
        const int64_t ws_pieces = (int64_t)((workspace_bytes - cpattn::kSchedBytes) / piece_bytes(D));
        const SplitPlan p = plan_split(a.BH, Sq, Skv, D, a.slots, (uint64_t)ws_pieces * piece_bytes(D));
        if (p.split_tiles > 0) {
            a.split_tiles = p.split_tiles;
            a.split_pieces = p.pieces;
            a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + cpattn::kSchedBytes);
            a.ws_lse = a.ws_o + (size_t)ws_pieces * cpattn::kAttnTileRows * D;
        }
    }
    return hip_status(cpattn::launch_attn_fwd_fp8(a));
}

CPATTN_EXPORT cpattn_status cpattn_attn_fwd_split_plan(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                                       int64_t slots, uint64_t workspace_bytes,
                                                       int64_t* split_tiles, int64_t* pieces,
                                                       uint64_t* bytes_used) {
    if (!split_tiles || !pieces || !bytes_used) return CPATTN_E_NULL;
    AttnCheck c;
    const cpattn_status st = check_attn_shapes(B, H, Sq, Skv, D, 1.0f, 32, &c);
    if (st != CPATTN_OK) return st;
    if (slots < 0 || slots > kMaxDim) return CPATTN_E_SHAPE;
    // the workspace starts with the dynamic schedule's counters; less than that is no workspace
    const bool sched = workspace_bytes >= (uint64_t)cpattn::kSchedBytes;
    const SplitPlan p = plan_split(B * H, Sq, Skv, D, slots, sched ? workspace_bytes - cpattn::kSchedBytes : 0);
    *split_tiles = p.split_tiles;
    *pieces = p.pieces;
    *bytes_used = sched ? p.bytes + cpattn::kSchedBytes : 0;
    return CPATTN_OK;
}

CPATTN_EXPORT cpattn_status cpattn_attn_fwd_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                                           int64_t D, cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                                                           uint64_t* bytes) {
    if (!bytes) return CPATTN_E_NULL;
    const int idt = enum_bits(in_dtype), odt = enum_bits(o_dtype);
    const bool fp8 = idt == CPATTN_E4M3;
    if ((!dtype_valid(idt) && !fp8) || !dtype_valid(odt)) return CPATTN_E_DTYPE;
    if (fp8 && odt != CPATTN_BF16 && odt != CPATTN_F32) return CPATTN_E_DTYPE;
    AttnCheck c;
    const cpattn_status st = check_attn_shapes(B, H, Sq, Skv, D, 1.0f, 32, &c);
    if (st != CPATTN_OK) return st;
    if (fp8 && D != 128) return CPATTN_E_HEADDIM;
    *bytes = 0;
    if (!dtype_16bit(idt) && !fp8) return CPATTN_OK;
    const int64_t slots = device_slots(D, odt == CPATTN_F32, fp8);
    if (slots <= 0) return CPATTN_E_HIP;
    *bytes = cpattn::kSchedBytes + plan_split(B * H, Sq, Skv, D, slots, UINT64_MAX).bytes;
    return CPATTN_OK;
}

CPATTN_EXPORT cpattn_status cpattn_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                                              const float* lse_b, void* o_out, float* lse_out, int64_t B,
                                              int64_t H, int64_t S, int64_t D, cpattn_dtype o_dtype,
                                              hipStream_t stream) {
    if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return CPATTN_E_NULL;
    const int odt = enum_bits(o_dtype);
    if (!dtype_valid(odt)) return CPATTN_E_DTYPE;
    if (!dims_ok({B, H, S}, 1)) return CPATTN_E_SHAPE;
    const int64_t osz = dtype_size(odt);
    if (D < 8 || D > 1024 || (D * osz) % 16 != 0) return CPATTN_E_HEADDIM;
    const int64_t rows = prod({B, H, S});
    const int64_t elems = prod({B, H, S, D});
    if (rows < 0 || elems < 0 || rows > (kMaxDim - 1) * 4) return CPATTN_E_SHAPE;
    // one launch holds fewer than 2^32 work-items
    if (cpattn::attn_merge_blocks(rows, D, merge_out(odt)) * 256 > (int64_t)UINT32_MAX) return CPATTN_E_SHAPE;
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
    cpattn::MergeArgs m{o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, D, merge_out(odt), stream};
    return hip_status(cpattn::launch_attn_merge(m));
}

CPATTN_EXPORT cpattn_status cpattn_ring_attn_fwd(const void* q, const void* k_chunks, const void* v_chunks,
                                                 float* o, float* lse, float* o_work, float* lse_work, int64_t B,
                                                 int64_t H, int64_t Sq, int64_t Skv_chunk, int64_t n_chunks,
                                                 int64_t D, float scale, hipStream_t stream) {
    if (!q || !o || !lse) return CPATTN_E_NULL;
    if (n_chunks < 1 || n_chunks > kMaxDim) return CPATTN_E_SHAPE;
    if (Skv_chunk != 0 && (!k_chunks || !v_chunks)) return CPATTN_E_NULL;
    if ((o_work == nullptr) != (lse_work == nullptr)) return CPATTN_E_NULL;
    AttnCheck c;
    const cpattn_status st = check_attn_shapes(B, H, Sq, Skv_chunk, D, scale, 32, &c);
    if (st != CPATTN_OK) return st;
    const int64_t all_kv = mul_checked(c.kv_elems, n_chunks);
    if (all_kv < 0) return CPATTN_E_SHAPE;
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse) ||
        (Skv_chunk && (!aligned16(k_chunks) || !aligned16(v_chunks))) ||
        (o_work && (!aligned16(o_work) || !aligned16(lse_work))))
        return CPATTN_E_ALIGN;
    const Range rq = range(q, c.q_elems * 2), rk = range(k_chunks, all_kv * 2), rv = range(v_chunks, all_kv * 2);
    const Range ro = range(o, c.q_elems * 4), rl = range(lse, c.rows * 4);
    const Range rw = o_work ? range(o_work, c.q_elems * 4) : Range{0, 0};
    const Range rlw = o_work ? range(lse_work, c.rows * 4) : Range{0, 0};
    const Range outs[4] = {ro, rl, rw, rlw};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], rq) || overlap(outs[i], rk) || overlap(outs[i], rv)) return CPATTN_E_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return CPATTN_E_ALIAS;
    }
    const int64_t chunk_bytes = c.kv_elems * 2;
    // The work buffers, when given, are the workspace: the dynamic schedule's counters take the
    // head of lse_work, and the key-range pieces of split tiles (one tile of rows each) take
    // o_work and the rest of lse_work.
    constexpr int64_t kSchedFloats = cpattn::kSchedBytes / 4;
    const bool work = o_work && lse_work && c.rows >= kSchedFloats;
    unsigned long long* sched = work ? reinterpret_cast<unsigned long long*>(lse_work) : nullptr;
    const int64_t ws_pieces =
        work ? std::min(c.rows / cpattn::kAttnTileRows, (c.rows - kSchedFloats) / cpattn::kAttnTileRows) : 0;
    float* ws_lse = work ? lse_work + kSchedFloats : nullptr;
    // Chunk c takes counter set c % kSchedSets; the launch of every kSchedSets-th chunk clears the
    // sets of that chunk and the next kSchedSets - 1 (one small kernel per 16 chunks).
    cpattn_status s = CPATTN_OK;
    for (int64_t ch = 0; ch < n_chunks && s == CPATTN_OK; ++ch) {
        const char* kc = static_cast<const char*>(k_chunks) + ch * chunk_bytes;
        const char* vc = static_cast<const char*>(v_chunks) + ch * chunk_bytes;
        const int64_t w = ch % cpattn::kSchedSets;
        s = run_attn(q, kc, vc, o, lse, B, H, Sq, Skv_chunk, D, scale, CPATTN_BF16, CPATTN_F32, ch > 0, false,
                     work ? o_work : nullptr, ws_lse, ws_pieces, sched ? sched + w * cpattn::kSchedSetWords : nullptr,
                     (sched && w == 0) ? sched : nullptr, stream);
    }
    return s;
}

namespace {

cpattn_status relayout(const void* const* srcs, void* const* dsts, int64_t n, int64_t B, int64_t S_local, int64_t H,
                       int64_t D, int64_t P, int dt, int dir, bool pack, hipStream_t stream) {
    if (!srcs || !dsts) return CPATTN_E_NULL;
    if (n < 1 || n > cpattn::kMaxRelayoutTensors) return CPATTN_E_SHAPE;
    for (int64_t i = 0; i < n; ++i)
        if (!srcs[i] || !dsts[i]) return CPATTN_E_NULL;
    if (!dtype_valid(dt)) return CPATTN_E_DTYPE;
    if (dir != CPATTN_SEQ_TO_HEAD && dir != CPATTN_HEAD_TO_SEQ) return CPATTN_E_SHAPE;
    if (!dims_ok({B, S_local, H, D, P}, 1) || H % P != 0) return CPATTN_E_SHAPE;
    const int64_t row_bytes = D * dtype_size(dt);
    if (row_bytes % 16 != 0) return CPATTN_E_HEADDIM;
    const int64_t n_rows = prod({B, S_local, H});
    const int64_t bytes = mul_checked(n_rows, row_bytes);
    // 32-bit row indices and 16-byte chunk indices within a row in the kernel (its grid strides
    // over tiles of rows, so their count is free)
    if (n_rows < 0 || bytes < 0 || n_rows > (int64_t)UINT32_MAX || row_bytes / 16 > (int64_t)INT32_MAX)
        return CPATTN_E_SHAPE;
    for (int64_t i = 0; i < n; ++i)
        if (!aligned16(srcs[i]) || !aligned16(dsts[i])) return CPATTN_E_ALIGN;
    // every destination is disjoint from every source and from every other destination
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j) {
            if (overlap(range(dsts[i], bytes), range(srcs[j], bytes))) return CPATTN_E_ALIAS;
            if (j != i && overlap(range(dsts[i], bytes), range(dsts[j], bytes))) return CPATTN_E_ALIAS;
        }
    const int mode = (dir == CPATTN_SEQ_TO_HEAD ? 0 : 2) + (pack ? 0 : 1);
    cpattn::RelayoutArgs a{};
    for (int64_t i = 0; i < n; ++i) {
        a.ptrs.src[i] = srcs[i];
        a.ptrs.dst[i] = dsts[i];
    }
    a.n_tensors = (int)n;
    a.B = B;
    a.S_local = S_local;
    a.H = H;
    a.P = P;
    a.row_bytes = row_bytes;
    a.mode = mode;
    a.stream = stream;
    return hip_status(cpattn::launch_relayout(a));
}

}  // namespace

CPATTN_EXPORT cpattn_status cpattn_ulysses_pack(const void* src, void* dst, int64_t B, int64_t S_local, int64_t H,
                                                int64_t D, int64_t P, cpattn_dtype dt, cpattn_dir dir,
                                                hipStream_t stream) {
    return relayout(&src, &dst, 1, B, S_local, H, D, P, enum_bits(dt), enum_bits(dir), true, stream);
}

CPATTN_EXPORT cpattn_status cpattn_ulysses_unpack(const void* src, void* dst, int64_t B, int64_t S_local,
                                                  int64_t H, int64_t D, int64_t P, cpattn_dtype dt,
                                                  cpattn_dir dir, hipStream_t stream) {
    return relayout(&src, &dst, 1, B, S_local, H, D, P, enum_bits(dt), enum_bits(dir), false, stream);
}

CPATTN_EXPORT cpattn_status cpattn_ulysses_pack_n(const void* const* srcs, void* const* dsts, int64_t n_tensors,
                                                  int64_t B, int64_t S_local, int64_t H, int64_t D, int64_t P,
                                                  cpattn_dtype dt, cpattn_dir dir, hipStream_t stream) {
    return relayout(srcs, dsts, n_tensors, B, S_local, H, D, P, enum_bits(dt), enum_bits(dir), true, stream);
}

CPATTN_EXPORT cpattn_status cpattn_ulysses_unpack_n(const void* const* srcs, void* const* dsts, int64_t n_tensors,
                                                    int64_t B, int64_t S_local, int64_t H, int64_t D, int64_t P,
                                                    cpattn_dtype dt, cpattn_dir dir, hipStream_t stream) {
    return relayout(srcs, dsts, n_tensors, B, S_local, H, D, P, enum_bits(dt), enum_bits(dir), false, stream);
}

namespace {

// Host-side rounding of a float to the 16-bit types (nearest, ties to even).
float round_to_f16_host(float x) { return (float)(_Float16)x; }
float round_to_bf16_host(float x) {
    uint32_t b;
    memcpy(&b, &x, 4);
    b = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
    float r;
    memcpy(&r, &b, 4);
    return r;
}

}  // namespace

CPATTN_EXPORT cpattn_status cpattn_qk_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int64_t D,
                                              float eps, float post_scale, cpattn_dtype dt, hipStream_t stream) {
    if (!x || !w || !y) return CPATTN_E_NULL;
    const int dtb = enum_bits(dt);
    if (!dtype_16bit(dtb)) return CPATTN_E_DTYPE;
    if (D < 8 || D > 512 || (D & (D - 1)) != 0) return CPATTN_E_HEADDIM;
    if (rows < 1 || rows > kMaxDim / (D / 8)) return CPATTN_E_SHAPE;   // one thread per 16 bytes
    if (!(eps >= 0.f) || !isfinite(eps) || !(post_scale > 0.f) || !isfinite(post_scale)) return CPATTN_E_SCALE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return CPATTN_E_ALIGN;
    const int64_t bytes = rows * D * 2;
    const Range rx = range(x, bytes), ry = range(y, bytes), rw = range(w, D * 2);
    if ((y != x && overlap(rx, ry)) || overlap(rw, ry)) return CPATTN_E_ALIAS;
    const bool f16 = dtb == CPATTN_F16;
    const float s16 = f16 ? round_to_f16_host(post_scale) : round_to_bf16_host(post_scale);
    if (!(s16 > 0.f) || !isfinite(s16)) return CPATTN_E_SCALE;   // underflows or overflows the 16-bit type
    cpattn::QkNormArgs a{x, w, y, rows, D, eps, s16, post_scale != 1.0f, f16, stream};
    return hip_status(cpattn::launch_qk_rmsnorm(a));
}

CPATTN_EXPORT const char* cpattn_status_string(cpattn_status s) {
    switch (enum_bits(s)) {
        case CPATTN_OK: return "ok";
        case CPATTN_E_NULL: return "a required pointer is NULL";
        case CPATTN_E_SHAPE: return "a size is out of range, inconsistent or overflows";
        case CPATTN_E_DTYPE: return "unsupported dtype or dtype combination";
        case CPATTN_E_HEADDIM: return "head dimension not supported";
        case CPATTN_E_ALIGN: return "a pointer is not 16-byte aligned";
        case CPATTN_E_ALIAS: return "buffers overlap where overlap is not allowed";
        case CPATTN_E_HIP: return "the HIP runtime rejected a launch";
        case CPATTN_E_SCALE: return "the score scale is not a finite positive number";
        case CPATTN_E_FLAGS: return "unknown flag bits";
    }
    return "unknown status";
}

CPATTN_EXPORT int cpattn_abi_version(void) { return CPATTN_ABI_VERSION; }
