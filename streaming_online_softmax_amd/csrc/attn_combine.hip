// attn_combine.hip -- LSE-weighted merge of a split-K workspace (Modular MAX
// "fa4_splitk_combine": per-row-head formulas, base 2 throughout, and its performance
// structure), written for wave64:
//   * one wave per output row-head, four row-heads per workgroup (fewer, larger workgroups to
//     dispatch); the row's depth is split into 16-byte lane slices, and 64 / (depth/4)
//     partitions are folded concurrently by separate lane groups;
//   * the LSE reduction (max, log-sum-exp, per-partition scale) is computed once into lane
//     registers: lane t holds partitions t, t+64, ...;
//   * each partition's scale reaches its lane group by a cross-lane read (ds_bpermute) for the
//     unrolled small-P instantiations, or from a 256-entry LDS table for the runtime-P one;
//   * loads run ahead of the FMAs: for the unrolled P every slice of the row-head is loaded
//     before the first is folded; for the runtime P the next slices are loaded before the
//     current ones are folded (software pipelining), so load latency overlaps the FMAs.
// An empty partition (lse = -inf) gets scale exactly 0; if every partition is empty the output
// is 0 and the LSE -inf (the all-masked convention of Tylo.jl "Register fragments and logical
// axes", section "Worked softmax", applied to the merge).
#include "device.h"
#include "launch.h"

namespace attn {

template <typename TO> struct out_store;
template <> struct out_store<float> {
  static __device__ __forceinline__ void put4(void* base, int64_t idx, f32x4 v) {
    *reinterpret_cast<f32x4*>((float*)base + idx) = v;
  }
};
template <> struct out_store<bf16_t> {
  static __device__ __forceinline__ void put4(void* base, int64_t idx, f32x4 v) {
    *reinterpret_cast<u32x2*>((uint16_t*)base + idx) = u32x2{elem<bf16_t>::pack2(v[0], v[1]), elem<bf16_t>::pack2(v[2], v[3])};
  }
};
template <> struct out_store<f16_t> {
  static __device__ __forceinline__ void put4(void* base, int64_t idx, f32x4 v) {
    *reinterpret_cast<u32x2*>((uint16_t*)base + idx) = u32x2{elem<f16_t>::pack2(v[0], v[1]), elem<f16_t>::pack2(v[2], v[3])};
  }
};

constexpr int kCombineWaves = 4;   // row-heads (waves) per workgroup

// The workspace is read exactly once: non-temporal (streaming) loads keep it from displacing
// other lines in the caches.
__device__ __forceinline__ f32x4 ld_stream(const float* a) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a));
}

template <int P_STATIC, int DEPTH, typename TO>
__global__ __launch_bounds__(64 * kCombineWaves) void attn_combine_kernel(CombineParams p) {
  constexpr int LPP = DEPTH / 4;              // lanes per partition slice (16 bytes each)
  constexpr int G = 64 / LPP;                 // partitions folded at once
  constexpr int NL = P_STATIC ? (P_STATIC + 63) / 64 : ATTN_P_MAX_DEV / 64;
  const int P = P_STATIC ? P_STATIC : p.P;

  __shared__ float sc_lds[P_STATIC ? 1 : kCombineWaves][P_STATIC ? 1 : ATTN_P_MAX_DEV];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t RH = p.RH;
  // a wave past the last row-head computes on row-head RH-1 and stores nothing (it still
  // reaches the workgroup barrier of the runtime-P path)
  const int64_t rh_w = (int64_t)blockIdx.x * kCombineWaves + wave;
  const bool live = rh_w < RH;
  const int64_t rh = live ? rh_w : RH - 1;

  // ---- LSE phase: once per row-head, into registers
  float ls[NL];
#pragma unroll
  for (int t = 0; t < NL; ++t) {
    const int pp = lane + 64 * t;
    ls[t] = pp < P ? p.lse_partial[(int64_t)pp * RH + rh] : kNegInf;
  }
  float mx = ls[0];
#pragma unroll
  for (int t = 1; t < NL; ++t) mx = fmaxf(mx, ls[t]);
  mx = across_groups_max<1>(mx);
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < NL; ++t) sum += (ls[t] == kNegInf) ? 0.f : fast_exp2(ls[t] - mx);
  sum = group_sum<64>(sum);
  const bool empty = (mx == kNegInf);
  const float Gl = empty ? kNegInf : log2f(sum) + mx;
  float sc[NL];
#pragma unroll
  for (int t = 0; t < NL; ++t) sc[t] = (empty || ls[t] == kNegInf) ? 0.f : fast_exp2(ls[t] - Gl);
  if constexpr (!P_STATIC) {
#pragma unroll
    for (int t = 0; t < NL; ++t) sc_lds[wave][lane + 64 * t] = sc[t];
    __syncthreads();   // orders each wave's table writes before its reads
  }

  // ---- weighted accumulation over partitions, next slice prefetched
  const int g = lane / LPP, dl = lane % LPP;
  const int64_t pstride = RH * DEPTH;
  const float* src = p.o_partial + rh * DEPTH + dl * 4;
  auto scale_of = [&](int pp) -> float {
    if constexpr (P_STATIC) {
      // pp < P_STATIC <= 64: partition pp lives in lane pp, register 0
      return __shfl(sc[0], pp < P ? pp : 0, 64) * (pp < P ? 1.f : 0.f);
    } else {
      return pp < P ? sc_lds[wave][pp] : 0.f;
    }
  };
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (P_STATIC) {
    constexpr int NS = (P_STATIC + G - 1) / G;   // slices per lane group
    f32x4 slice[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int pp = i * G + g;
      slice[i] = pp < P ? ld_stream(src + (int64_t)pp * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float s = scale_of(i * G + g);
      acc += (s != 0.f) ? s * slice[i] : f32x4{0.f, 0.f, 0.f, 0.f};   // an empty partition adds nothing
    }
  } else {
    f32x4 cur = g < P ? ld_stream(src + (int64_t)g * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int pp0 = 0; pp0 < P; pp0 += G) {
      const int pn = pp0 + G + g;
      f32x4 nxt = pn < P ? ld_stream(src + (int64_t)pn * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
      const float s = scale_of(pp0 + g);
      acc += (s != 0.f) ? s * cur : f32x4{0.f, 0.f, 0.f, 0.f};   // an empty partition adds nothing
      cur = nxt;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = across_groups_sum<LPP>(acc[j]);
  if (live && g == 0) out_store<TO>::put4(p.out, rh * DEPTH + dl * 4, acc);
  if (live && lane == 0 && p.lse_out) p.lse_out[rh] = empty ? kNegInf : Gl * kLn2;
}

template <int P_STATIC, int DEPTH>
static hipError_t launch_combine_t(const CombineParams& p, int out_dtype, hipStream_t s) {
  dim3 grid((unsigned)((p.RH + kCombineWaves - 1) / kCombineWaves));
  dim3 block(64 * kCombineWaves);
  if (out_dtype == 2) hipLaunchKernelGGL((attn_combine_kernel<P_STATIC, DEPTH, float>), grid, block, 0, s, p);
  else if (out_dtype == 0) hipLaunchKernelGGL((attn_combine_kernel<P_STATIC, DEPTH, bf16_t>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_combine_kernel<P_STATIC, DEPTH, f16_t>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <int DEPTH>
static hipError_t launch_combine_depth(const CombineParams& p, int out_dtype, hipStream_t s) {
  switch (p.P) {
    case 4: return launch_combine_t<4, DEPTH>(p, out_dtype, s);
    case 8: return launch_combine_t<8, DEPTH>(p, out_dtype, s);
    case 16: return launch_combine_t<16, DEPTH>(p, out_dtype, s);
    default: return launch_combine_t<0, DEPTH>(p, out_dtype, s);
  }
}

hipError_t launch_combine(const CombineParams& p, int depth, int out_dtype, hipStream_t s) {
  switch (depth) {
    case 16: return launch_combine_depth<16>(p, out_dtype, s);
    case 32: return launch_combine_depth<32>(p, out_dtype, s);
    case 64: return launch_combine_depth<64>(p, out_dtype, s);
    case 128: return launch_combine_depth<128>(p, out_dtype, s);
    case 256: return launch_combine_depth<256>(p, out_dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
