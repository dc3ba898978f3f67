// layout_probe.hip -- TEST INFRASTRUCTURE: one-wave probe kernels that run the device helpers of
// streaming_online_softmax_amd/csrc/device.h (and the raw gfx950 instructions the attention
// kernels build on) on inputs supplied by the test, so that every lane / register map the kernels
// assume can be compared with its written-down form.  The pages ask for exactly this kind of
// check of register correspondences: coordinate tests that enumerate every lane and value, and a
// GPU test that compares the register path with a store / load through shared memory and
// consumes the result in a second matrix product (Tylo.jl "Streaming attention and online
// state", section "Same-lane conversion").
//
// Every entry point takes device pointers of the sizes stated, launches one 64-lane workgroup
// on the default stream and returns the HIP status of the launch.
#include "../../streaming_online_softmax_amd/csrc/device.h"

using namespace attn;

namespace {

// a, b: 64 lanes x 4 u32 (8 bf16 per lane, lane-major); c: 64 lanes x 16 f32
__global__ void k_mfma_bf16(const u32x4* a, const u32x4* b, float* c) {
  const int l = threadIdx.x;
  const f32x16 acc = elem<bf16_t>::mfma32(a[l], b[l], f32x16{});
  for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

// a, b: 64 lanes x 8 i32 (32 E4M3 bytes per lane); c: 64 lanes x 16 f32
__global__ void k_mfma_f8(const i32x8* a, const i32x8* b, float* c) {
  const int l = threadIdx.x;
  const f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], f32x16{}, 0, 0, 0, 0, 0, 0);
  for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

// fill: 2048 u16 staged into LDS; addr: 64 byte offsets (multiples of 8, addr + 8 <= 4096);
// out: 64 lanes x 4 u16
__global__ void k_tr16(const uint16_t* fill, const int* addr, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2048];
  for (int i = threadIdx.x; i < 2048; i += 64) lds[i] = fill[i];
  __syncthreads();
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((uint8_t*)lds + addr[threadIdx.x]));
  for (int j = 0; j < 4; ++j) out[threadIdx.x * 4 + j] = (uint16_t)v[j];
}

// fill: 4096 bytes staged into LDS; addr as above; out: 64 lanes x 8 bytes
__global__ void k_tr8(const uint8_t* fill, const int* addr, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4096];
  for (int i = threadIdx.x; i < 4096; i += 64) lds[i] = fill[i];
  __syncthreads();
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds + addr[threadIdx.x]));
  for (int j = 0; j < 8; ++j) out[threadIdx.x * 8 + j] = (uint8_t)(((uint32_t)v[j / 4]) >> (8 * (j % 4)));
}

// x: 64 floats; out: 64 lanes x 4 (xor32_sum, xor32_max, xor16_sum, group_sum<64>)
__global__ void k_xlane(const float* x, float* out) {
  const int l = threadIdx.x;
  const float v = x[l];
  out[l * 4 + 0] = xor32_sum(v);
  out[l * 4 + 1] = xor32_max(v);
  out[l * 4 + 2] = xor16_sum(v);
  out[l * 4 + 3] = group_sum<64>(v);
}

// The same-lane conversion of the attention kernels on one 32-key block (D = 16 for the first
// product, 32 output rows for the second), computed two ways:
//   register path: S^T = K_pi Q^T with K rows in key_perm order, the 16 score registers packed
//   pairwise to bf16 in place as the two B operands of O^T = V^T P^T;
//   LDS path: the same scores stored to LDS at their logical (key, query) coordinates from the
//   accumulator map, read back at the B-operand coordinates of the second product, packed.
// k: [32 keys][16] bf16, q: [32 queries][16] bf16, v: [32 keys][32] bf16 (raw u16);
// o_reg, o_lds: 64 lanes x 16 f32 (O^T accumulators of the two paths); s: [32][32] f32 scores
__global__ void k_same_lane(const uint16_t* k, const uint16_t* q, const uint16_t* v, float* o_reg,
                            float* o_lds, float* s) {
  __shared__ float sl[32][33];
  const int l = threadIdx.x, half = l >> 5, col = l & 31;
  u32x4 a, bq;
  {
    const int key = key_perm(col);
    uint16_t ka[8], qa[8];
    for (int j = 0; j < 8; ++j) { ka[j] = k[key * 16 + 8 * half + j]; qa[j] = q[col * 16 + 8 * half + j]; }
    for (int j = 0; j < 4; ++j) {
      a[j] = (uint32_t)ka[2 * j] | ((uint32_t)ka[2 * j + 1] << 16);
      bq[j] = (uint32_t)qa[2 * j] | ((uint32_t)qa[2 * j + 1] << 16);
    }
  }
  const f32x16 st = elem<bf16_t>::mfma32(a, bq, f32x16{});
  // V^T as the A operand of the second product for key step k2: lane holds V[16 k2 + 8 half + j][col]
  u32x4 va[2];
  for (int k2 = 0; k2 < 2; ++k2)
    for (int j = 0; j < 4; ++j)
      va[k2][j] = (uint32_t)v[(16 * k2 + 8 * half + 2 * j) * 32 + col] |
                  ((uint32_t)v[(16 * k2 + 8 * half + 2 * j + 1) * 32 + col] << 16);
  // register path
  f32x16 o1 = f32x16{};
  for (int k2 = 0; k2 < 2; ++k2) {
    u32x4 pb;
    for (int i = 0; i < 4; ++i) pb[i] = elem<bf16_t>::pack2(st[8 * k2 + 2 * i], st[8 * k2 + 2 * i + 1]);
    o1 = elem<bf16_t>::mfma32(va[k2], pb, o1);
  }
  // LDS path: accumulator register r holds S^T[row (r/4)*8 + 4 half + r%4][col], row = pi position
  for (int r = 0; r < 16; ++r) sl[key_perm((r / 4) * 8 + 4 * half + (r % 4))][col] = st[r];
  __syncthreads();
  f32x16 o2 = f32x16{};
  for (int k2 = 0; k2 < 2; ++k2) {
    u32x4 pb;
    for (int i = 0; i < 4; ++i)
      pb[i] = elem<bf16_t>::pack2(sl[16 * k2 + 8 * half + 2 * i][col], sl[16 * k2 + 8 * half + 2 * i + 1][col]);
    o2 = elem<bf16_t>::mfma32(va[k2], pb, o2);
  }
  for (int r = 0; r < 16; ++r) { o_reg[l * 16 + r] = o1[r]; o_lds[l * 16 + r] = o2[r]; }
  for (int i = l; i < 1024; i += 64) s[i] = sl[i / 32][i % 32];
}

}  // namespace

extern "C" {
int probe_mfma_bf16(const void* a, const void* b, float* c) {
  hipLaunchKernelGGL(k_mfma_bf16, dim3(1), dim3(64), 0, 0, (const u32x4*)a, (const u32x4*)b, c);
  return (int)hipGetLastError();
}
int probe_mfma_f8(const void* a, const void* b, float* c) {
  hipLaunchKernelGGL(k_mfma_f8, dim3(1), dim3(64), 0, 0, (const i32x8*)a, (const i32x8*)b, c);
  return (int)hipGetLastError();
}
int probe_tr16(const void* fill, const int* addr, void* out) {
  hipLaunchKernelGGL(k_tr16, dim3(1), dim3(64), 0, 0, (const uint16_t*)fill, addr, (uint16_t*)out);
  return (int)hipGetLastError();
}
int probe_tr8(const void* fill, const int* addr, void* out) {
  hipLaunchKernelGGL(k_tr8, dim3(1), dim3(64), 0, 0, (const uint8_t*)fill, addr, (uint8_t*)out);
  return (int)hipGetLastError();
}
int probe_xlane(const float* x, float* out) {
  hipLaunchKernelGGL(k_xlane, dim3(1), dim3(64), 0, 0, x, out);
  return (int)hipGetLastError();
}
int probe_same_lane(const void* k, const void* q, const void* v, float* o_reg, float* o_lds, float* s) {
  hipLaunchKernelGGL(k_same_lane, dim3(1), dim3(64), 0, 0, (const uint16_t*)k, (const uint16_t*)q,
                     (const uint16_t*)v, o_reg, o_lds, s);
  return (int)hipGetLastError();
}
}
