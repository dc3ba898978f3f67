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

hipError_t launch_round(const float* x, void* y, int64_t n, int dtype, hipStream_t s) {
  const int64_t pairs = n / 2;
  int64_t blocks = (pairs + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;              // grid-stride beyond 2M pairs
  if (dtype == 0)
    round_kernel<bf16_t><<<(unsigned)blocks, 256, 0, s>>>(x, (uint16_t*)y, n);
  else
    round_kernel<f16_t><<<(unsigned)blocks, 256, 0, s>>>(x, (uint16_t*)y, n);
  return hipGetLastError();
}

}  // namespace attn
