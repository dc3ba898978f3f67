// attn_combine.hip -- LSE-weighted merge of a split-K workspace (Modular MAX
// "fa4_splitk_combine": per-row-head formulas, base 2 throughout, and its performance
// structure), written for wave64:
//   * one wave per output row-head (four per workgroup when there are many row-heads), or, when
//     there are few row-heads, the depth of each split over up to eight waves in workgroups of
//     one, so that a small merge reaches ~1024 waves on the 256 compute units; a wave's depth
//     slice is split into 16-byte lane slices, and 64 / (slice/4) partitions are folded side by
//     side by separate lane groups;
//   * each row-head's maximum, log-sum-exp and per-partition scales are reduced a single time,
//     into lane registers: lane t holds partitions t, t+64, ...;
//   * each partition's scale reaches its lane group by a cross-lane read (ds_bpermute) when
//     P <= 64, or from a 256-entry LDS table beyond;
//   * loads run ahead of the arithmetic: the first chunk of slices (16 per lane group) is issued
//     before the LSE loads, so their two memory round trips overlap, and every further chunk is
//     issued before the previous one is folded.  P up to 64 runs the instantiation of the next
//     power of two at or above it (4, 8, 16, 32, 64) with loads past P predicated off, so an
//     off-rung P such as 37 keeps the unrolled structure; larger P takes the same chunked loop
//     with a run-time trip count.
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

// The workspace is read exactly once: non-temporal (streaming) loads keep it from displacing
// other lines in the caches.
__device__ __forceinline__ f32x4 ld_stream(const float* a) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a));
}

constexpr int kCombineChunk = 16;   // slices per lane group per chunk of loads

// RUNG: the instantiation serves 1 <= P <= RUNG (RUNG = 4, 8, 16, 32 or 64), or any P up to
// ATTN_P_MAX_DEV when RUNG = 0.  DW: elements of the row-head's depth one wave merges (the
// depth, or a power-of-two part of it).  WAVES waves per workgroup.
template <int RUNG, int DW, typename TO, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void attn_combine_kernel(CombineParams p) {
  constexpr int LPP = DW / 4;                 // lanes per partition slice (16 bytes each)
  constexpr int G = 64 / LPP;                 // partitions folded side by side
  constexpr int NL = RUNG ? (RUNG + 63) / 64 : ATTN_P_MAX_DEV / 64;   // LSE registers per lane
  constexpr int NS = RUNG ? (RUNG + G - 1) / G : 0;                  // slices per lane group
  constexpr int CHS = (RUNG && NS < kCombineChunk) ? NS : kCombineChunk;   // slices per chunk
  constexpr bool SHFL = RUNG != 0 && RUNG <= 64;   // partition pp's scale sits in lane pp
  const int P = p.P;

  __shared__ float sc_lds[SHFL ? 1 : WAVES][SHFL ? 1 : ATTN_P_MAX_DEV];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t RH = p.RH;
  const int depth = p.depth;
  const int nsplit = depth / DW;              // waves per row-head
  // a wave past the last row-head computes on row-head RH-1 and stores nothing
  const int64_t w_all = (int64_t)blockIdx.x * WAVES + wave;
  const int64_t rh_w = w_all / nsplit;
  const int ds = (int)(w_all - rh_w * nsplit);   // this wave's depth slice
  const bool live = rh_w < RH;
  const int64_t rh = live ? rh_w : RH - 1;

  const int g = lane / LPP, dl = lane % LPP;
  const int64_t pstride = RH * depth;
  const int64_t col = rh * depth + ds * DW + dl * 4;   // first of this lane's four elements
  const float* src = p.o_partial + col;
  // slice i of chunk c of this lane group holds partition (c * CHS + i) * G + g
  auto load_chunk = [&](int c, f32x4 (&buf)[CHS]) {
#pragma unroll
    for (int i = 0; i < CHS; ++i) {
      const int pp = (c * CHS + i) * G + g;
      buf[i] = pp < P ? ld_stream(src + (int64_t)pp * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  f32x4 buf_a[CHS], buf_b[CHS];
  load_chunk(0, buf_a);   // in flight during the LSE phase

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
  if constexpr (!SHFL) {
    // the wave writes and then reads its own row of the table: LDS operations of one wave
    // complete in order, so only the compiler must keep the reads after the writes
#pragma unroll
    for (int t = 0; t < NL; ++t) sc_lds[wave][lane + 64 * t] = sc[t];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  auto scale_of = [&](int pp) -> float {
    if constexpr (SHFL) return __shfl(sc[0], pp < P ? pp : 0, 64) * (pp < P ? 1.f : 0.f);
    else return pp < P ? sc_lds[wave][pp] : 0.f;
  };

  // ---- weighted accumulation over the partitions, one chunk of slices ahead
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto fold_chunk = [&](int c, const f32x4 (&buf)[CHS]) {
#pragma unroll
    for (int i = 0; i < CHS; ++i) {
      const float s = scale_of((c * CHS + i) * G + g);
      acc += (s != 0.f) ? s * buf[i] : f32x4{0.f, 0.f, 0.f, 0.f};   // an empty partition adds nothing
    }
  };
  auto two_chunks = [&](int c, int nch) {
    if (c + 1 < nch) load_chunk(c + 1, buf_b);
    fold_chunk(c, buf_a);
    if (c + 1 < nch) {
      if (c + 2 < nch) load_chunk(c + 2, buf_a);
      fold_chunk(c + 1, buf_b);
    }
  };
  if constexpr (RUNG != 0) {
    constexpr int NCH = (NS + CHS - 1) / CHS;
#pragma unroll
    for (int c = 0; c < NCH; c += 2) two_chunks(c, NCH);
  } else {
    const int nch = ((P + G - 1) / G + CHS - 1) / CHS;
    for (int c = 0; c < nch; c += 2) two_chunks(c, nch);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = across_groups_sum<LPP>(acc[j]);
  if (live && g == 0) out_store<TO>::put4(p.out, col, acc);
  if (live && ds == 0 && lane == 0 && p.lse_out) p.lse_out[rh] = empty ? kNegInf : Gl * kLn2;
}

// Waves per workgroup: four when the launch has enough waves to give every compute unit several
// workgroups, else one (a decode-sized merge then spreads over more compute units).
constexpr int64_t kCombineManyWaves = 4 * 1024;
// Few row-heads: split each row-head's depth until the launch has this many waves.
constexpr int64_t kCombineTargetWaves = 1024;

template <int RUNG, int DW, typename TO>
static void launch_combine_w(const CombineParams& p, hipStream_t s) {
  const int64_t waves = p.RH * (p.depth / DW);
  if (waves >= kCombineManyWaves)
    hipLaunchKernelGGL((attn_combine_kernel<RUNG, DW, TO, 4>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_combine_kernel<RUNG, DW, TO, 1>), dim3((unsigned)waves), dim3(64), 0, s, p);
}

template <int RUNG, typename TO>
static hipError_t launch_combine_dw(const CombineParams& p, hipStream_t s) {
  int nsplit = 1;   // waves per row-head: a power of two, slices of at least 16 elements
  while (nsplit < 8 && p.depth / (2 * nsplit) >= 16 && p.RH * nsplit < kCombineTargetWaves) nsplit *= 2;
  switch (p.depth / nsplit) {
    case 16: launch_combine_w<RUNG, 16, TO>(p, s); break;
    case 32: launch_combine_w<RUNG, 32, TO>(p, s); break;
    case 64: launch_combine_w<RUNG, 64, TO>(p, s); break;
    case 128: launch_combine_w<RUNG, 128, TO>(p, s); break;
    case 256: launch_combine_w<RUNG, 256, TO>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int RUNG>
static hipError_t launch_combine_t(const CombineParams& p, int out_dtype, hipStream_t s) {
  if (out_dtype == 2) return launch_combine_dw<RUNG, float>(p, s);
  if (out_dtype == 0) return launch_combine_dw<RUNG, bf16_t>(p, s);
  return launch_combine_dw<RUNG, f16_t>(p, s);
}

hipError_t launch_combine(const CombineParams& p0, int depth, int out_dtype, hipStream_t s) {
  if (depth != 16 && depth != 32 && depth != 64 && depth != 128 && depth != 256) return hipErrorInvalidValue;
  CombineParams p = p0;
  p.depth = depth;
  if (p.P <= 4) return launch_combine_t<4>(p, out_dtype, s);
  if (p.P <= 8) return launch_combine_t<8>(p, out_dtype, s);
  if (p.P <= 16) return launch_combine_t<16>(p, out_dtype, s);
  if (p.P <= 32) return launch_combine_t<32>(p, out_dtype, s);
  if (p.P <= 64) return launch_combine_t<64>(p, out_dtype, s);
  return launch_combine_t<0>(p, out_dtype, s);
}

}  // namespace attn
