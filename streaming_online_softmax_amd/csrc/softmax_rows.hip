// softmax_rows.hip -- standalone row softmax y = softmax(x) along each row of a row-major
// [rows, n] array, with the all-masked conventions of Tylo.jl "Register fragments and logical
// axes", section "Worked softmax": a logit of -inf is a masked entry (weight 0), and a row whose
// logits are all -inf gives zeros, never NaN.
//
// Three kernels, the three the Tylo page "Streaming attention and online state" (section
// "Online statistics") compares:
//   STREAM  two passes, four values per lane per step regardless of the row width: the first
//           pass streams the running statistics (m, l) -- the online update of the same section
//           -- each lane over its own elements, merged across the wave once at the end; the
//           second pass rereads the logits and writes the probabilities.  Registers do not grow
//           with n.
//   REGS    the whole row in registers: one read, one write.  Up to 4096 elements one wave holds
//           the row; beyond that (up to 65536) a workgroup of 16 waves holds it and the two row
//           reductions cross the waves once each through LDS.
//   THREE   a scalar three-pass loop (max, sum of exponentials, write), one value per lane.
// One wave owns one row, so every reduction stays inside the wave.  Exponentials are taken in
// base 2 of (logit - reference) * log2(e).  Rows are processed four to a workgroup (one per wave).
#include "device.h"
#include "launch.h"

namespace attn {

// element access: 4 consecutive elements as floats, and the rounding store back.  The
// probabilities are written once and never reread here, so they are stored non-temporally; a
// load marked LAST is the final read of those logits (it need not stay in the caches).
template <typename T> __device__ __forceinline__ T ld_nt_if(const T* a, bool nt) {
  return nt ? __builtin_nontemporal_load(a) : *a;
}
template <typename TE> struct sm_io;
template <> struct sm_io<float> {
  template <bool LAST = false>
  static __device__ __forceinline__ f32x4 load4(const void* base, int64_t i) {
    return ld_nt_if(reinterpret_cast<const f32x4*>((const float*)base + i), LAST);
  }
  static __device__ __forceinline__ float load1(const void* base, int64_t i) { return ((const float*)base)[i]; }
  static __device__ __forceinline__ void store4(void* base, int64_t i, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>((float*)base + i));
  }
  static __device__ __forceinline__ void store1(void* base, int64_t i, float v) { ((float*)base)[i] = v; }
};
template <typename T16> struct sm_io16 {
  using E = elem<T16>;
  template <bool LAST = false>
  static __device__ __forceinline__ f32x4 load4(const void* base, int64_t i) {
    const u32x2 w = ld_nt_if(reinterpret_cast<const u32x2*>((const uint16_t*)base + i), LAST);
    return f32x4{E::to_f32((uint16_t)(w[0] & 0xFFFFu)), E::to_f32((uint16_t)(w[0] >> 16)),
                 E::to_f32((uint16_t)(w[1] & 0xFFFFu)), E::to_f32((uint16_t)(w[1] >> 16))};
  }
  static __device__ __forceinline__ float load1(const void* base, int64_t i) {
    return E::to_f32(((const uint16_t*)base)[i]);
  }
  static __device__ __forceinline__ void store4(void* base, int64_t i, f32x4 v) {
    __builtin_nontemporal_store(u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])}, reinterpret_cast<u32x2*>((uint16_t*)base + i));
  }
  static __device__ __forceinline__ void store1(void* base, int64_t i, float v) {
    ((uint16_t*)base)[i] = (uint16_t)(E::pack2(v, 0.f) & 0xFFFFu);
  }
};
template <> struct sm_io<bf16_t> : sm_io16<bf16_t> {};
template <> struct sm_io<f16_t> : sm_io16<f16_t> {};

// weight of logit x against the reference m: 2^((x - m) log2 e).  The difference is taken
// first, so the rounding error scales with |x - m| (small for every weight that matters), not
// with |x| as in x log2e - m log2e.  A masked logit (-inf) gives 0; callers never pass a -inf
// reference (all-masked rows are finished separately).
__device__ __forceinline__ float sm_weight(float x, float m) { return fast_exp2((x - m) * kLog2e); }

// Merge of lane-local (max, sum) summaries over the wave (Tylo "Online statistics": merge of
// two summaries, each sum rescaled to the common maximum; an empty summary (-inf, 0) adds 0).
__device__ __forceinline__ void sm_wave_merge(float& m, float& l) {
  const float M = across_groups_max<1>(m);
  float ls = (m == kNegInf) ? 0.f : l * fast_exp2((m - M) * kLog2e);
  l = group_sum<64>(ls);
  m = M;
}

constexpr int kSmRegsMax = 16;   // REGS: up to 16 steps of 4 values per lane (n <= 4096)
constexpr int kSmWideWaves = 16; // REGS beyond 4096: 16 waves per row, up to 16 steps (n <= 65536)

template <typename TE, int METHOD, bool VEC, int R>
__global__ __launch_bounds__(256) void softmax_rows_kernel(SoftmaxParams p) {
  using IO = sm_io<TE>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= p.rows) return;                       // wave-uniform
  const int n = p.n;
  const int64_t base = row * (int64_t)n;

  if constexpr (METHOD == SM_STREAM) {
    // ---- pass 1: lane-local online statistics over 4-value steps, then one wave merge
    float m = kNegInf, l = 0.f;
    auto absorb = [&](f32x4 v) {
      const float cm = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
      const float mn = fmaxf(m, cm);
      if (mn != kNegInf) {
        const float alpha = (m == kNegInf) ? 0.f : sm_weight(m, mn);
        l = alpha * l + ((sm_weight(v[0], mn) + sm_weight(v[1], mn)) + (sm_weight(v[2], mn) + sm_weight(v[3], mn)));
        m = mn;
      }
    };
    const int nv = VEC ? (n & ~3) : 0;             // elements covered by 4-value steps
    constexpr int U = 4;                           // steps in flight per lane
    int j = 4 * lane;
    for (; j + 256 * (U - 1) < nv; j += 256 * U) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = IO::load4(p.x, base + j + 256 * u);
#pragma unroll
      for (int u = 0; u < U; ++u) absorb(v[u]);
    }
    for (; j < nv; j += 256) absorb(IO::load4(p.x, base + j));
    for (int t = nv + lane; t < n; t += 64) {      // tail (or every element when not vectorised)
      const float x = IO::load1(p.x, base + t);
      absorb(f32x4{x, kNegInf, kNegInf, kNegInf});
    }
    sm_wave_merge(m, l);
    // ---- pass 2: reread, normalise (all-masked row: zeros)
    const bool empty = (m == kNegInf);
    const float mref = empty ? 0.f : m;   // the reference (finite)
    const float inv = empty ? 0.f : 1.f / l;
    j = 4 * lane;
    for (; j + 256 * (U - 1) < nv; j += 256 * U) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = IO::template load4<true>(p.x, base + j + 256 * u);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = sm_weight(v[u][e], mref) * inv;
        IO::store4(p.y, base + j + 256 * u, y);
      }
    }
    for (; j < nv; j += 256) {
      const f32x4 v = IO::template load4<true>(p.x, base + j);
      f32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = sm_weight(v[e], mref) * inv;
      IO::store4(p.y, base + j, y);
    }
    for (int t = nv + lane; t < n; t += 64) IO::store1(p.y, base + t, sm_weight(IO::load1(p.x, base + t), mref) * inv);
  } else if constexpr (METHOD == SM_REGS) {
    // ---- the whole row in registers: R steps of 4 values per lane (missing entries: -inf)
    f32x4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = 256 * r + 4 * lane;
      if (VEC && j + 3 < n) {
        v[r] = IO::template load4<true>(p.x, base + j);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[r][e] = (j + e < n) ? IO::load1(p.x, base + j + e) : kNegInf;
      }
    }
    float m = kNegInf;
#pragma unroll
    for (int r = 0; r < R; ++r) m = fmaxf(m, fmaxf(fmaxf(v[r][0], v[r][1]), fmaxf(v[r][2], v[r][3])));
    m = across_groups_max<1>(m);
    const bool empty = (m == kNegInf);
    const float mref = empty ? 0.f : m;   // the reference (finite)
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[r][e] = empty ? 0.f : sm_weight(v[r][e], mref);
        l += v[r][e];
      }
    l = group_sum<64>(l);
    const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = 256 * r + 4 * lane;
      const f32x4 y = v[r] * inv;
      if (VEC && j + 3 < n) {
        IO::store4(p.y, base + j, y);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) if (j + e < n) IO::store1(p.y, base + j + e, y[e]);
      }
    }
  } else {
    // ---- scalar three-pass loop: max, sum of exponentials, write
    float m = kNegInf;
    for (int t = lane; t < n; t += 64) m = fmaxf(m, IO::load1(p.x, base + t));
    m = across_groups_max<1>(m);
    const bool empty = (m == kNegInf);
    const float mref = empty ? 0.f : m;   // the reference (finite)
    float l = 0.f;
    if (!empty)
      for (int t = lane; t < n; t += 64) l += sm_weight(IO::load1(p.x, base + t), mref);
    l = group_sum<64>(l);
    const float inv = empty ? 0.f : 1.f / l;
    for (int t = lane; t < n; t += 64) IO::store1(p.y, base + t, sm_weight(IO::load1(p.x, base + t), mref) * inv);
  }
}

// REGS for wide rows: one workgroup of kSmWideWaves waves per row.  Thread t holds elements
// 4 (1024 r + t) .. +3 for r < R (16-byte accesses, consecutive threads contiguous); the row max
// and the row sum are each reduced in the wave, then across the waves through LDS (every thread
// folds the 16 wave values in the same order).
template <typename TE, bool VEC, int R>
__global__ __launch_bounds__(64 * kSmWideWaves) void softmax_rows_wide_kernel(SoftmaxParams p) {
  using IO = sm_io<TE>;
  constexpr int NT = 64 * kSmWideWaves;
  __shared__ float red[2][kSmWideWaves];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = p.n;
  const int64_t base = (int64_t)blockIdx.x * n;
  f32x4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = 4 * (NT * r + t);
    if (VEC && j + 3 < n) {
      v[r] = IO::template load4<true>(p.x, base + j);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[r][e] = (j + e < n) ? IO::load1(p.x, base + j + e) : kNegInf;
    }
  }
  float m = kNegInf;
#pragma unroll
  for (int r = 0; r < R; ++r) m = fmaxf(m, fmaxf(fmaxf(v[r][0], v[r][1]), fmaxf(v[r][2], v[r][3])));
  m = across_groups_max<1>(m);
  if (lane == 0) red[0][wave] = m;
  __syncthreads();
  m = red[0][0];
#pragma unroll
  for (int w = 1; w < kSmWideWaves; ++w) m = fmaxf(m, red[0][w]);
  const bool empty = (m == kNegInf);
  const float mref = empty ? 0.f : m;   // the reference (finite)
  float l = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[r][e] = empty ? 0.f : sm_weight(v[r][e], mref);
      l += v[r][e];
    }
  l = group_sum<64>(l);
  if (lane == 0) red[1][wave] = l;
  __syncthreads();
  l = red[1][0];
#pragma unroll
  for (int w = 1; w < kSmWideWaves; ++w) l += red[1][w];
  const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = 4 * (NT * r + t);
    const f32x4 y = v[r] * inv;
    if (VEC && j + 3 < n) {
      IO::store4(p.y, base + j, y);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) if (j + e < n) IO::store1(p.y, base + j + e, y[e]);
    }
  }
}

template <typename TE, int METHOD, bool VEC>
static hipError_t launch_sm_t(const SoftmaxParams& p, hipStream_t s) {
  dim3 grid((unsigned)((p.rows + 3) / 4));
  if constexpr (METHOD == SM_REGS) {
    if (p.n > 256 * kSmRegsMax) {                  // a workgroup per row
      const dim3 g2((unsigned)p.rows), b2(64 * kSmWideWaves);
      const int wsteps = (p.n + 4 * 64 * kSmWideWaves - 1) / (4 * 64 * kSmWideWaves);
      if (wsteps <= 2) hipLaunchKernelGGL((softmax_rows_wide_kernel<TE, VEC, 2>), g2, b2, 0, s, p);
      else if (wsteps <= 4) hipLaunchKernelGGL((softmax_rows_wide_kernel<TE, VEC, 4>), g2, b2, 0, s, p);
      else if (wsteps <= 8) hipLaunchKernelGGL((softmax_rows_wide_kernel<TE, VEC, 8>), g2, b2, 0, s, p);
      else hipLaunchKernelGGL((softmax_rows_wide_kernel<TE, VEC, kSmRegsMax>), g2, b2, 0, s, p);
      return hipGetLastError();
    }
    const int steps = (p.n + 255) / 256;
    if (steps <= 1) hipLaunchKernelGGL((softmax_rows_kernel<TE, METHOD, VEC, 1>), grid, dim3(256), 0, s, p);
    else if (steps <= 2) hipLaunchKernelGGL((softmax_rows_kernel<TE, METHOD, VEC, 2>), grid, dim3(256), 0, s, p);
    else if (steps <= 4) hipLaunchKernelGGL((softmax_rows_kernel<TE, METHOD, VEC, 4>), grid, dim3(256), 0, s, p);
    else if (steps <= 8) hipLaunchKernelGGL((softmax_rows_kernel<TE, METHOD, VEC, 8>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((softmax_rows_kernel<TE, METHOD, VEC, kSmRegsMax>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((softmax_rows_kernel<TE, METHOD, VEC, 1>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <typename TE, int METHOD>
static hipError_t launch_sm_vec(const SoftmaxParams& p, bool vec, hipStream_t s) {
  return vec ? launch_sm_t<TE, METHOD, true>(p, s) : launch_sm_t<TE, METHOD, false>(p, s);
}

template <typename TE>
static hipError_t launch_sm_method(const SoftmaxParams& p, int method, bool vec, hipStream_t s) {
  switch (method) {
    case SM_STREAM: return launch_sm_vec<TE, SM_STREAM>(p, vec, s);
    case SM_REGS: return launch_sm_vec<TE, SM_REGS>(p, vec, s);
    case SM_THREE: return launch_sm_vec<TE, SM_THREE>(p, vec, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_softmax_rows(const SoftmaxParams& p, int dtype, int method, bool vec, hipStream_t s) {
  if (dtype == 0) return launch_sm_method<bf16_t>(p, method, vec, s);
  if (dtype == 1) return launch_sm_method<f16_t>(p, method, vec, s);
  return launch_sm_method<float>(p, method, vec, s);
}

int softmax_regs_max_n() { return 4 * 64 * kSmWideWaves * kSmRegsMax; }   // 65536

}  // namespace attn
