// Internal launcher interface between the C ABI (api.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

struct AttnFwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t BH;      // B * H
    int64_t Sq;
    int64_t Skv;     // >= 1 (Skv == 0 is handled by launch_fill_empty)
    int64_t D;       // 64 or 128
    float scale;
    bool out_f32;
    hipStream_t stream;
};

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a);
hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a);

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
    bool f32;        // o dtype: f32 if true, bf16 otherwise
    hipStream_t stream;
};

hipError_t launch_attn_merge(const MergeArgs& a);

// Relayout modes (see cpattn.h): 0 pack seq->head, 1 unpack seq->head,
// 2 pack head->seq, 3 unpack head->seq.
struct RelayoutArgs {
    const void* src;
    void* dst;
    int64_t B, S_local, H, P;
    int64_t row_bytes;   // D * element size, a multiple of 16
    int mode;
    hipStream_t stream;
};

hipError_t launch_relayout(const RelayoutArgs& a);

}  // namespace cpattn
