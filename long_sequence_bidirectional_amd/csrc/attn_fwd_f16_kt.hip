// fp16 instantiations of the matrix-core attention kernel with K stored sequence-last
// (attn_fwd_kernel.h), in a unit of their own so the units build in parallel.
#include "attn_fwd_kernel.h"

namespace cpattn {

hipError_t launch_attn_fwd_f16_kt(const AttnFwdArgs& a) { return launch_kt<true>(a); }

}  // namespace cpattn
