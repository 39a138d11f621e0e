// fp16 instantiations of the matrix-core attention kernel (attn_fwd_kernel.h).
#include "attn_fwd_kernel.h"

namespace cpattn {

hipError_t launch_attn_fwd_f16(const AttnFwdArgs& a) { return launch_any<true>(a); }

}  // namespace cpattn
