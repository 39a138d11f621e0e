// bf16 instantiations of the matrix-core attention kernel (attn_fwd_kernel.h).
#include "attn_fwd_kernel.h"

namespace cpattn {

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a) { return launch_any<false>(a); }

int attn_fwd_bf16_blocks_per_cu(int64_t D, bool out_f32) {
    if (D == 128) return out_f32 ? occupancy<128, false, true>() : occupancy<128, false, false>();
    return out_f32 ? occupancy<64, false, true>() : occupancy<64, false, false>();
}

}  // namespace cpattn
