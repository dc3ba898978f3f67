// convert.hip -- FP32 -> bf16 / fp16 rounding through the same packed conversion the attention
// kernels apply to the probabilities before the second product and to the stored output
// (Tylo.jl "Streaming attention and online state", section "Same-lane conversion": round to
// nearest even, no saturation or flush to zero; Tylo.jl "Register fragments and logical axes",
// section "Logical types and register packing": the packed word, low element in the low half).
// Exposed so that the conversion itself can be compared bit for bit with a reference.
#include "device.h"
#include "launch.h"

namespace attn {

// Thread i converts the pair (x[2i], x[2i+1]) with one packed conversion and stores one 32-bit
// word; an odd tail element is converted as the low half of a pair and stored alone.
template <typename T>
__global__ __launch_bounds__(256) void round_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n) {
  const int64_t pairs = n / 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pairs; i += stride) {
    const uint32_t w = elem<T>::pack2(x[2 * i], x[2 * i + 1]);
    y[2 * i] = (uint16_t)(w & 0xffffu);
    y[2 * i + 1] = (uint16_t)(w >> 16);
  }
  if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0) y[n - 1] = (uint16_t)(elem<T>::pack2(x[n - 1], 0.0f) & 0xffffu);
}

// E4M3: the kernels' packed conversion (v_cvt_pk_fp8_f32: round to nearest even; beyond the
// largest finite value it gives NaN) preceded by a clamp to +-448, which makes it saturate as the
// pages' 8-bit conversion does (Tylo.jl "Register fragments and logical axes", section "Logical
// types and register packing"): values in (448, 464] round to 448 either way, larger ones and
// infinities clamp to 448; comparisons with NaN are false, so NaN passes to the conversion and
// stays NaN.  Probabilities never need the clamp (they are at most 256).
__device__ __forceinline__ float sat_e4m3(float x) { return x > 448.f ? 448.f : (x < -448.f ? -448.f : x); }

__global__ __launch_bounds__(256) void round_fp8_kernel(const float* __restrict__ x, uint8_t* __restrict__ y, int64_t n) {
  const int64_t pairs = n / 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pairs; i += stride) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(x[2 * i]), sat_e4m3(x[2 * i + 1]), 0, false);
    y[2 * i] = (uint8_t)(w & 0xff);
    y[2 * i + 1] = (uint8_t)((w >> 8) & 0xff);
  }
  if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0)
    y[n - 1] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(x[n - 1]), 0.f, 0, false) & 0xff);
}

hipError_t launch_round(const float* x, void* y, int64_t n, int dtype, hipStream_t s) {
  const int64_t pairs = n / 2;
  int64_t blocks = (pairs + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;              // grid-stride beyond 2M pairs
  if (dtype == 0)
    round_kernel<bf16_t><<<(unsigned)blocks, 256, 0, s>>>(x, (uint16_t*)y, n);
  else if (dtype == 1)
    round_kernel<f16_t><<<(unsigned)blocks, 256, 0, s>>>(x, (uint16_t*)y, n);
  else
    round_fp8_kernel<<<(unsigned)blocks, 256, 0, s>>>(x, (uint8_t*)y, n);
  return hipGetLastError();
}

}  // namespace attn
