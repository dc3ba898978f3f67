// mask_pack.hip -- a byte mask re-encoded as one bit per (query, key) in the register order of
// the attention kernels (the mask's meaning: triton-cuda-lab workshop "A3. Tiled attention with
// online normalization", section "Masks that preserve the recurrence"; the encoding is this
// library's).  The matrix-core kernels hold the scores of 32 query rows x 32 keys as 16
// registers per lane: register r of lane l is row l % 32, key 16 (r / 8) + 8 (l / 32) + r % 8.
// One 32-bit word per lane then covers the lane's scores of 64 keys (two such blocks), so a
// kernel reads 256 contiguous bytes per wave and 64 keys instead of 2 KiB of mask rows.
#include "device.h"
#include "launch.h"

namespace attn {

// Bit e (0..7) set iff byte e of x is nonzero.  Per byte, adding 0x7f to its low seven bits
// carries into bit 7 iff they are nonzero; OR-ing x's own bit 7 then marks every nonzero byte.
// The multiply gathers the four marks of a 32-bit half into bits 21..24 (shifted copies at
// 0, 7, 14 and 21 places never overlap, so nothing carries).
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t x) {
  const uint32_t t = ((((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u) >> 7;
  return ((t * 0x00204081u) >> 21) & 0xfu;
}

// One wave per (row group g, key group c), four key groups per workgroup; lane l assembles word
// (g, c, l).  Its row's keys 64 c + 16 j + 8 (l / 32) .. +8 (j = 0..3) go to bits 8 j .. 8 j + 7.
__global__ __launch_bounds__(256) void mask_pack_kernel(const uint8_t* __restrict__ mask, int Nq, int Nkv,
                                                        int causal, int vec, int n_kg, int n_cb,
                                                        uint32_t* __restrict__ bits) {
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x / n_cb;
  const int c = (blockIdx.x % n_cb) * 4 + (threadIdx.x >> 6);
  if (c >= n_kg) return;
  if (causal && 64 * c > 32 * g + 31) return;   // no key of the group is visible to these rows
  const int row = 32 * g + (lane & 31);
  uint32_t word = 0;
  if (row < Nq) {
    const uint8_t* mrow = mask + (int64_t)row * Nkv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key0 = 64 * c + 16 * j + 8 * (lane >> 5);
      uint32_t b8 = 0;
      if (vec && key0 + 8 <= Nkv) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(mrow + key0);
        b8 = nonzero_bytes4(x[0]) | (nonzero_bytes4(x[1]) << 4);
      } else {
        for (int e = 0; e < 8; ++e)
          if (key0 + e < Nkv && mrow[key0 + e] != 0) b8 |= 1u << e;
      }
      word |= b8 << (8 * j);
    }
  }
  bits[((int64_t)g * n_kg + c) * 64 + lane] = word;
}

hipError_t launch_mask_pack(const uint8_t* mask, int Nq, int Nkv, int causal, uint32_t* bits, hipStream_t s) {
  const int n_g = (Nq + 31) / 32, n_kg = (Nkv + 63) / 64, n_cb = (n_kg + 3) / 4;
  const int vec = ((uintptr_t)mask % 8 == 0) && (Nkv % 8 == 0);
  const int64_t blocks = (int64_t)n_g * n_cb;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  mask_pack_kernel<<<(unsigned)blocks, 256, 0, s>>>(mask, Nq, Nkv, causal, vec, n_kg, n_cb, bits);
  return hipGetLastError();
}

}  // namespace attn
