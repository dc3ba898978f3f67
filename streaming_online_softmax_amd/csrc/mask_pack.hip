// mask_pack.hip -- a byte mask re-encoded as one bit per (query, key) in the register order of
// the attention kernels (the mask's meaning: triton-cuda-lab workshop "A3. Tiled attention with
// online normalization", section "Masks that preserve the recurrence"; the encoding is this
// library's).  The matrix-core kernels hold the scores of 32 query rows x 32 keys as 16
// registers per lane: register r of lane l is row l % 32, key 16 (r / 8) + 8 (l / 32) + r % 8.
// One 32-bit word per lane then covers the lane's scores of 64 keys (two such blocks), so a
// kernel reads 256 contiguous bytes per wave and 64 keys instead of 2 KiB of mask rows.
// Bit e (0..15) of a 16-byte chunk's code is byte e being nonzero.
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

// One workgroup per 32-row group g and 4 key groups (256 keys): the rows' 256-byte spans are
// read in 16-byte chunks, consecutive threads taking consecutive chunks of a row, and each
// chunk's nonzero bytes become 16 bits in LDS.  Wave w then assembles the words of key group
// 4 cb + w: lane l takes row l % 32 and, for j = 0..3, bits 8 (l / 32) .. +8 of chunk 4 w + j
// (keys 64 c + 16 j + 8 (l / 32) .. +8) as its bits 8 j .. 8 j + 7.
__global__ __launch_bounds__(256) void mask_pack_kernel(const uint8_t* __restrict__ mask, int Nq, int Nkv,
                                                        int causal, int vec, int n_kg, int n_cb,
                                                        uint32_t* __restrict__ bits) {
  __shared__ uint16_t nz[32][16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = blockIdx.x / n_cb, cb = blockIdx.x % n_cb;
  if (causal && 256 * cb > 32 * g + 31) return;   // every key group of the workgroup above the diagonal
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = t + 256 * s, r = i >> 4, ch = i & 15;
    const int row = 32 * g + r, key0 = 256 * cb + 16 * ch;
    uint32_t b16 = 0;
    if (row < Nq && key0 < Nkv) {
      const uint8_t* src = mask + (int64_t)row * Nkv + key0;
      if (vec && key0 + 16 <= Nkv) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(src);
        b16 = nonzero_bytes4(x[0]) | (nonzero_bytes4(x[1]) << 4) | (nonzero_bytes4(x[2]) << 8) |
              (nonzero_bytes4(x[3]) << 12);
      } else {
        for (int e = 0; e < 16; ++e)
          if (key0 + e < Nkv && src[e] != 0) b16 |= 1u << e;
      }
    }
    nz[r][ch] = (uint16_t)b16;
  }
  __syncthreads();
  const int c = 4 * cb + wave;
  if (c >= n_kg || (causal && 64 * c > 32 * g + 31)) return;   // no key of the group is visible to these rows
  const int r = lane & 31, h = lane >> 5;
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) word |= ((uint32_t)(nz[r][4 * wave + j] >> (8 * h)) & 0xffu) << (8 * j);
  bits[((int64_t)g * n_kg + c) * 64 + lane] = word;
}

hipError_t launch_mask_pack(const uint8_t* mask, int Nq, int Nkv, int causal, uint32_t* bits, hipStream_t s) {
  const int n_g = (Nq + 31) / 32, n_kg = (Nkv + 63) / 64, n_cb = (n_kg + 3) / 4;
  const int vec = ((uintptr_t)mask % 16 == 0) && (Nkv % 16 == 0);   // every row start 16-byte aligned
  const int64_t blocks = (int64_t)n_g * n_cb;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  mask_pack_kernel<<<(unsigned)blocks, 256, 0, s>>>(mask, Nq, Nkv, causal, vec, n_kg, n_cb, bits);
  return hipGetLastError();
}

}  // namespace attn
