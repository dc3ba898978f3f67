// device.h -- gfx950 device helpers shared by the attention kernels.
//
// Matrix-core operand layouts used below (v_mfma_f32_32x32x16_{bf16,f16}, wave64, verified on
// gfx950 by enumerating every lane and register against a host product):
//   A (32 x 16):  lane l holds A[l % 32][(l / 32) * 8 + j],   j = 0..7
//   B (16 x 32):  lane l holds B[(l / 32) * 8 + j][l % 32],   j = 0..7
//   C (32 x 32):  lane l, register r holds C[(r / 4) * 8 + (l / 32) * 4 + (r % 4)][l % 32]
// ds_read_b64_tr_b16 (per 16-lane group): lane i receives, for j = 0..3, element (i % 4) of the
// 8-byte chunk addressed by lane 4 * j + i / 4 of its group.
// global_load_lds_dwordx4 writes lane l's 16 bytes at LDS base + 16 * l (a wave-instruction
// fills 1 KiB contiguously); its immediate offset is added to both addresses.
// v_permlane32_swap(x, x) returns (x_lo32 | x_lo32, x_hi32 | x_hi32) as a pair, so combining the
// pair gives the xor-32 reduction in every lane; v_permlane16_swap does the same for xor 16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ------------------------------------------------------------------------------------------
// Element types.  Storage is raw 16-bit words; conversions round to nearest even (the
// hardware conversions v_cvt_pk_bf16_f32 and v_cvt_pk_f16_f32 under the default rounding mode,
// checked on gfx950 against an independent RNE reference including ties, subnormals, signed
// zero, infinities and overflow).
// ------------------------------------------------------------------------------------------
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

template <typename T> struct elem;
template <> struct elem<bf16_t> {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
  // one v_cvt_pk_bf16_f32: lo in bits 15:0, hi in bits 31:16
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  }
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct elem<f16_t> {
  typedef f16x8 vec8;
  static __device__ __forceinline__ float to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
  // one v_cvt_pk_f16_f32 (round to nearest even, subnormals kept)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
  }
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// Row permutation of a 32-key block inside the first product S^T = K Q^T: A-operand row i holds
// key pi(i).  With it, accumulator register r of lane l holds key 16*(r/8) + 8*(l/32) + (r%8),
// which is exactly the B-operand slot order of the second product for key step r/8, so the
// scores convert to that operand in the lanes that hold them.
__device__ __forceinline__ int key_perm(int i) {
  int b = i >> 3, h = (i >> 2) & 1;
  return ((b >> 1) << 4) + (h << 3) + ((b & 1) << 2) + (i & 3);
}

// ------------------------------------------------------------------------------------------
// Cross-lane reductions (all 64 lanes take part; results replicated in every lane involved).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float xor32_max(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP moves inside a 16-lane row.
enum : int {
  DPP_QUAD_XOR1 = 0xB1,    // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,    // quad_perm [2,3,0,1]
  DPP_ROW_MIRROR = 0x140,  // lane i <- 15 - i
  DPP_ROW_HALF_MIRROR = 0x141  // lane i <- 7 - i within each half row
};
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W consecutive lanes (W = 1..64, a power of two); the result is
// bitwise identical in every lane of a group (each step adds a commutative pair).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (W >= 2) x = x + dpp<DPP_QUAD_XOR1>(x);
  if constexpr (W >= 4) x = x + dpp<DPP_QUAD_XOR2>(x);
  if constexpr (W >= 8) x = x + dpp<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (W >= 16) x = x + dpp<DPP_ROW_MIRROR>(x);
  if constexpr (W >= 32) x = xor16_sum(x);
  if constexpr (W >= 64) x = xor32_sum(x);
  return x;
}

// xor-shuffle inside 32-lane halves through ds_swizzle's bitmask mode (and 0x1f, xor MASK).
template <int MASK>
__device__ __forceinline__ float swz_xor(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (MASK << 10) | 0x1F));
}

// Max / sum over the lanes that share (lane % W) -- i.e. across the 64 / W groups of W lanes.
// Every step combines a lane with its xor partner, so the result is bitwise identical in all
// lanes of a residue class.
template <int W>
__device__ __forceinline__ float across_groups_max(float x) {
  if constexpr (W <= 1) { x = fmaxf(x, dpp<DPP_QUAD_XOR1>(x)); }
  if constexpr (W <= 2) { x = fmaxf(x, dpp<DPP_QUAD_XOR2>(x)); }
  if constexpr (W <= 4) { x = fmaxf(x, swz_xor<4>(x)); }
  if constexpr (W <= 8) { x = fmaxf(x, swz_xor<8>(x)); }
  if constexpr (W <= 16) { x = xor16_max(x); }
  if constexpr (W <= 32) { x = xor32_max(x); }
  return x;
}
template <int W>
__device__ __forceinline__ float across_groups_sum(float x) {
  if constexpr (W <= 1) { x = x + dpp<DPP_QUAD_XOR1>(x); }
  if constexpr (W <= 2) { x = x + dpp<DPP_QUAD_XOR2>(x); }
  if constexpr (W <= 4) { x = x + swz_xor<4>(x); }
  if constexpr (W <= 8) { x = x + swz_xor<8>(x); }
  if constexpr (W <= 16) { x = xor16_sum(x); }
  if constexpr (W <= 32) { x = xor32_sum(x); }
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace attn
