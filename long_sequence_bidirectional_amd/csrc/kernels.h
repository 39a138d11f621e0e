// Internal launcher interface between the C ABI (api.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// Query rows per workgroup tile of the bf16 attention kernel.
constexpr int kAttnTileRows = 256;

// Element strides of an attention operand: element (b, h, s, d) sits at
// b * batch + h * head + s * row + d.  Head-major [B,H,S,D]: row = D,
// head = S*D; sequence-major [B,S,H,D]: row = H*D, head = D.
struct Strides {
    int64_t batch, head, row;
};

struct AttnFwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t BH;      // B * H
    int64_t H;
    bool seq_major;        // operands [B,S,H,D] (else [B,H,S,D]); the strides below agree
    bool k_seq_last;       // k is [B,H,D,Skv] (q, v, o head-major; 16-bit inputs, Skv % 8 == 0)
    Strides sq, skv, so;   // of q, of k and v, of o (lse is always [B, H, Sq])
    int64_t Sq;
    int64_t Skv;     // >= 1 (Skv == 0 is handled by launch_fill_empty)
    int64_t D;       // 64 or 128
    float scale;
    bool out_f32;
    bool accumulate;       // fold into the (O, LSE) already in o/lse (out_f32 only)
    // Key-range split of the last split_tiles tiles into split_pieces pieces each
    // (bf16 kernel only; 0 = none).  Partials go to ws_o [split_tiles * split_pieces,
    // kAttnTileRows, D] and ws_lse [split_tiles * split_pieces, kAttnTileRows] (f32) and
    // are merged into o/lse by launch_merge_pieces.
    int64_t split_tiles;
    int64_t split_pieces;
    float* ws_o;
    float* ws_lse;
    // Workgroups of the 16-bit kernel resident at once on the current device (0 = unknown):
    // the kernel is launched with at most that many workgroups, each looping over work units.
    int64_t slots;
    // Counter set of the dynamic unit schedule (kSchedSetWords words of device memory that are
    // zero when the kernel starts), or null for the static schedule.  sched_clear, when not null,
    // is the first of kSchedWords words (sched among them) that the launcher clears with a small
    // kernel before the attention kernel; null when the caller cleared sched already (the ring
    // driver clears the sets of up to kSchedSets chunks with one launch).
    unsigned long long* sched;
    unsigned long long* sched_clear;
    hipStream_t stream;
};

// The dynamic schedule's counters: one set of kSchedSetWords words per launch (word x < 8 serves
// XCD x's own range of units, word 8 the shared tail), kSchedSets sets at the start of a
// workspace (a ring of launches takes one set each before they are cleared again).
constexpr int kSchedSetWords = 16;
constexpr int kSchedSets = 16;
constexpr int kSchedWords = kSchedSetWords * kSchedSets;
constexpr int kSchedBytes = kSchedWords * 8;

// Kernel-side form of the work split (passed by value).
struct AttnTileMap {
    int n_dp, per_xcd_dp, grid_dp;      // whole tiles [0, n_dp)
    int n_split, split_s, per_xcd_sp;   // split tiles [n_dp, n_dp + n_split), split_s pieces each
    float* ws_o;
    float* ws_lse;
    int accumulate;
    unsigned long long* sched;          // dynamic schedule's counter set, or null
    int per_xcd;                        // units [x*per_xcd, (x+1)*per_xcd) form XCD x's range
};

// Size of each XCD's own range of units under the dynamic schedule, for n_dp whole tiles and a
// grid of G workgroups (a multiple of the XCD count).  The ranges hold whole rounds of whole
// tiles (G per round), as many as fit in 7/8 of them and at least one; the rest of the whole
// tiles and every split piece (a fraction of a tile's work) form the tail shared by all XCDs, so
// the ranges carry equal work.  0 (no ranges, every unit from the shared counter) when the whole
// tiles do not fill one round.
inline int sched_per_xcd(int64_t n_dp, int64_t G) {
    const int64_t gx = G / 8;
    if (gx <= 0 || n_dp < G) return 0;
    const int64_t rounds = n_dp * 7 / (8 * G);
    return (int)(gx * (rounds > 1 ? rounds : 1));
}

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a);
hipError_t launch_attn_fwd_f16(const AttnFwdArgs& a);
hipError_t launch_attn_fwd_bf16_kt(const AttnFwdArgs& a);   // a.k_seq_last
hipError_t launch_attn_fwd_f16_kt(const AttnFwdArgs& a);
hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a);

// Attention with OCP FP8 E4M3 inputs (D = 128), one f32 scale per tensor.  Work split,
// split pieces, accumulation and schedule as in AttnFwdArgs.
struct AttnFp8Args {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t BH, H, Sq, Skv;
    bool seq_major;
    Strides sq, skv, so;
    float scale, q_scale, k_scale, v_scale;
    bool out_f32;            // O in f32 (else bf16)
    bool accumulate;         // fold into the (O, LSE) already in o/lse (out_f32 only)
    int64_t split_tiles;
    int64_t split_pieces;
    float* ws_o;
    float* ws_lse;
    int64_t slots;
    unsigned long long* sched;
    unsigned long long* sched_clear;
    hipStream_t stream;
};

hipError_t launch_attn_fwd_fp8(const AttnFp8Args& a);

// Resident workgroups per CU of the fp8 attention kernel (0 if the runtime cannot tell).
int attn_fwd_fp8_blocks_per_cu(bool out_f32);

// Resident workgroups per CU of the bf16 attention kernel (0 if the runtime cannot tell).
int attn_fwd_bf16_blocks_per_cu(int64_t D, bool out_f32);

// Storage type of a merged O.
enum class MergeOut { BF16, F16, F32 };

// Merge of the key-range pieces of split tiles (and, when accumulating, of the
// (O, LSE) already in o/lse) into the final rows of o/lse.
struct MergePiecesArgs {
    const float* ws_o;
    const float* ws_lse;
    void* o;
    float* lse;
    int first_tile;   // tile index of split tile 0
    int n_split;
    int pieces;
    int nQt;          // tiles per (b, h)
    int64_t H;
    Strides so;       // of o
    int64_t Sq;
    int64_t D;
    MergeOut out;
    bool accumulate;
    hipStream_t stream;
};

hipError_t launch_merge_pieces(const MergePiecesArgs& a);

// O = 0 (n_o elements of elem_bytes each), LSE = -inf (n_rows floats).
hipError_t launch_fill_empty(void* o, int64_t o_bytes, float* lse, int64_t n_rows, hipStream_t stream);

struct MergeArgs {
    const void* o_a;
    const float* lse_a;
    const void* o_b;
    const float* lse_b;
    void* o_out;
    float* lse_out;
    int64_t rows;    // B * H * S
    int64_t D;
    MergeOut o_type;
    hipStream_t stream;
};

hipError_t launch_attn_merge(const MergeArgs& a);

// Workgroups (256 work-items each) launch_attn_merge uses for `rows` rows of D values of type t.
// A launch holds fewer than 2^32 work-items, so the entry point refuses shapes with
// attn_merge_blocks(...) * 256 >= 2^32.
int64_t attn_merge_blocks(int64_t rows, int64_t D, MergeOut t);

// RMSNorm over rows of D 16-bit values, times w, rounded to the 16-bit type, then
// (has_scale) times the 16-bit constant scale16 and rounded again.
struct QkNormArgs {
    const void* x;
    const void* w;      // [D]
    void* y;            // may be x
    int64_t rows;
    int64_t D;          // power of two, 8..512
    float eps;
    float scale16;      // already a value of the 16-bit type
    bool has_scale;
    bool f16;           // fp16 (else bf16)
    hipStream_t stream;
};

hipError_t launch_qk_rmsnorm(const QkNormArgs& a);

// Relayout modes (see cpattn.h): 0 pack seq->head, 1 unpack seq->head,
// 2 pack head->seq, 3 unpack head->seq.
constexpr int kMaxRelayoutTensors = 8;
struct RelayoutPtrs {                 // passed to the kernel by value
    const void* src[kMaxRelayoutTensors];
    void* dst[kMaxRelayoutTensors];
};
struct RelayoutArgs {
    RelayoutPtrs ptrs;   // the first n_tensors entries are used
    int n_tensors;       // 1 .. kMaxRelayoutTensors, all of the same shape
    int64_t B, S_local, H, P;
    int64_t row_bytes;   // D * element size, a multiple of 16
    int mode;
    hipStream_t stream;
};

hipError_t launch_relayout(const RelayoutArgs& a);

}  // namespace cpattn
