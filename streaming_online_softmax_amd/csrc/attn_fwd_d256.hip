// attn_fwd_d256.hip -- the D = 256 instantiations of the attention forward kernel
// (attn_fwd_kernel.h), in a translation unit of their own so they can be built with the
// scheduling flags that suit them (one wave per SIMD, every register in use).
#include "attn_fwd_kernel.h"

namespace attn {

hipError_t launch_fwd_d256(const FwdParams& p, int dtype, bool split, hipStream_t s) {
  return dtype == 0 ? launch_fwd_mask<bf16_t, 256, 64>(p, split, s) : launch_fwd_mask<f16_t, 256, 64>(p, split, s);
}

}  // namespace attn
