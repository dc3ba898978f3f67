// attn_fwd.hip -- host dispatch of the attention forward kernel (attn_fwd_kernel.h) for
// D <= 128 and the FP8-V form; D = 256 is instantiated in attn_fwd_d256.hip.
#include "attn_fwd_kernel.h"

namespace attn {

template <typename T>
static hipError_t launch_fwd_dtype(const FwdParams& p, int D, int BN, bool split, hipStream_t s) {
  switch (D) {
    case 16: return BN == 32 ? launch_fwd_mask<T, 16, 32>(p, split, s) : launch_fwd_mask<T, 16, 64>(p, split, s);
    case 32: return BN == 32 ? launch_fwd_mask<T, 32, 32>(p, split, s) : launch_fwd_mask<T, 32, 64>(p, split, s);
    case 64: return BN == 32 ? launch_fwd_mask<T, 64, 32>(p, split, s) : launch_fwd_mask<T, 64, 64>(p, split, s);
    case 128: return launch_fwd_mask<T, 128, 64>(p, split, s);
    case 256: return launch_fwd_d256(p, std::is_same<T, bf16_t>::value ? 0 : 1, split, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int BN, bool split, hipStream_t s) {
  return dtype == 0 ? launch_fwd_dtype<bf16_t>(p, D, BN, split, s) : launch_fwd_dtype<f16_t>(p, D, BN, split, s);
}

template <typename T, int MASK, int FMT>
static hipError_t launch_fwd_v8_t(const FwdParams& p, hipStream_t s) {
  return launch_fwd_t<T, 128, 128, MASK, false, 8, FMT>(p, s);
}

template <typename T, int FMT>
static hipError_t launch_fwd_v8_mask(const FwdParams& p, hipStream_t s) {
  if (p.mask == nullptr) return launch_fwd_v8_t<T, kMaskNone, FMT>(p, s);
  return p.mask_lds ? launch_fwd_v8_t<T, kMaskLds, FMT>(p, s) : launch_fwd_v8_t<T, kMaskGlobal, FMT>(p, s);
}

hipError_t launch_fwd_fp8v(const FwdParams& p, int dtype, int v_format, hipStream_t s) {
  if (dtype == 0) return v_format == 1 ? launch_fwd_v8_mask<bf16_t, 2>(p, s) : launch_fwd_v8_mask<bf16_t, 1>(p, s);
  return v_format == 1 ? launch_fwd_v8_mask<f16_t, 2>(p, s) : launch_fwd_v8_mask<f16_t, 1>(p, s);
}

int fwd_block_m() { return kMinBlockM; }

}  // namespace attn
