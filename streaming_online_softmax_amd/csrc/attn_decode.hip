// attn_decode.hip -- split-K producer for few-query (decode) shapes: each workgroup streams one
// key partition of one row-head and writes the partition's locally normalised O_p / l_p and its
// base-2 log-sum-exp (Modular MAX "fa4_splitk_combine", workspace layout).
//
// With one query per head the work is a stream over K and V at about one FLOP per byte, so the
// kernel is built for HBM bandwidth, not for the matrix cores: D/8 lanes read one 16-byte slice
// each of a key row (a whole row per lane group, 64 / (D/8) rows per wave load), eight such
// loads of K and of V are in flight per lane, and the dot products are finished with in-row DPP
// adds.  The online-softmax recurrence (triton-cuda-lab workshop "A3. Tiled attention with
// online normalization", section "Keep three quantities for each query row") runs per 8-key
// step in log2 units; the four waves of a workgroup hold independent states over interleaved
// key chunks and are merged once at the end with the same rescale rule (Tylo.jl "Streaming
// attention and online state", section "Online statistics", merge of two summaries).
//
// Fused form (FUSED): after writing its workspace entry, each workgroup takes a ticket from its
// row-head's counter (one counter per 128-byte line: counters sharing a line serialise their
// atomics); the one that takes the last ticket merges all P entries with the LSE-weighted
// combine (Modular MAX "fa4_splitk_combine", per-row-head formulas) and writes the output, so
// decode is one launch instead of producer + combine.  This is the one-GPU stand-in for the
// page's programmatic launch overlap of the combine with the producer's tail.
#include "device.h"
#include "launch.h"

namespace attn {

// K and V are streamed once per (row-head, partition): non-temporal loads keep them from
// displacing reusable lines in the caches (measured +11% bandwidth at the decode shape).
__device__ __forceinline__ u32x4 ld_stream16(const uint16_t* a) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
}

// Workspace access.  The fused form publishes entries across workgroups of one launch, which
// may run on different XCDs: it uses device-coherent (agent-scope) stores and loads.
template <bool COHERENT>
__device__ __forceinline__ void put_ws(float* a, float x) {
  if constexpr (COHERENT) __hip_atomic_store(a, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *a = x;
}
__device__ __forceinline__ float get_ws(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int D, bool MASK, bool FUSED>
__global__ __launch_bounds__(256) void attn_decode_kernel(DecodeParams p) {
  using E = elem<T>;
  constexpr int LPK = D / 8;        // lanes per key row (16 bytes each)
  constexpr int KPW = 64 / LPK;     // key rows per wave load
  constexpr int U = 8;              // loads of K (and of V) in flight per lane
  constexpr int KPI = U * KPW;      // keys per wave iteration

  __shared__ float sm_m[4], sm_l[4];
  __shared__ __attribute__((aligned(16))) float sm_o[4][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane / LPK;         // key slot inside a wave load
  const int dl = lane % LPK;        // 8-element slice of the row

  int bid = blockIdx.x;
  const int part = bid % p.P;
  const int64_t rh = bid / p.P;     // (b * Nq + i) * H + h
  const int h = (int)(rh % p.H);
  const int64_t tok = rh / p.H;
  const int i = (int)(tok % p.Nq);
  const int b = (int)(tok / p.Nq);

  const int kbeg = part * p.chunk;
  int kend = min(kbeg + p.chunk, p.Nkv);
  if (p.causal) kend = min(kend, i + 1);

  const int64_t row_stride = (int64_t)p.H * D;
  const uint16_t* kbase = (const uint16_t*)p.k + ((int64_t)b * p.Nkv * p.H + h) * D + dl * 8;
  const uint16_t* vbase = (const uint16_t*)p.v + ((int64_t)b * p.Nkv * p.H + h) * D + dl * 8;
  const uint8_t* mrow = MASK ? p.mask + (int64_t)i * p.Nkv : nullptr;

  float qv[8];
  {
    u32x4 w = ld16((const uint16_t*)p.q + rh * D + dl * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qv[2 * j] = E::to_f32((uint16_t)(w[j] & 0xFFFFu));
      qv[2 * j + 1] = E::to_f32((uint16_t)(w[j] >> 16));
    }
  }
  const float c = p.scale_log2;

  float m_run = kNegInf, l_run = 0.f;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.f;

  for (int base = kbeg + wave * KPI; base < kend; base += 4 * KPI) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int key = base + u * KPW + g;
      key = key < p.Nkv ? key : p.Nkv - 1;
      kr[u] = ld_stream16(kbase + (int64_t)key * row_stride);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int key = base + u * KPW + g;
      key = key < p.Nkv ? key : p.Nkv - 1;
      vr[u] = ld_stream16(vbase + (int64_t)key * row_stride);
    }
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(qv[2 * j], E::to_f32((uint16_t)(kr[u][j] & 0xFFFFu)), acc);
        acc = fmaf(qv[2 * j + 1], E::to_f32((uint16_t)(kr[u][j] >> 16)), acc);
      }
      acc = group_sum<LPK>(acc);
      const int key = base + u * KPW + g;
      bool vis = key < kend;
      if constexpr (MASK) vis = vis && (mrow[key < p.Nkv ? key : 0] != 0);
      s[u] = vis ? acc : kNegInf;
    }
    float mx = s[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u]);
    mx = across_groups_max<LPK>(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = fast_exp2(fmaf(s[u], c, -m_use));
      psum += pu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = fmaf(pu, E::to_f32((uint16_t)(vr[u][j] & 0xFFFFu)), o[2 * j]);
        o[2 * j + 1] = fmaf(pu, E::to_f32((uint16_t)(vr[u][j] >> 16)), o[2 * j + 1]);
      }
    }
    l_run = alpha * l_run + psum;
  }

  // fold the key slots of the wave (same running max in every lane of a wave)
  l_run = across_groups_sum<LPK>(l_run);
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = across_groups_sum<LPK>(o[j]);
  if (g == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sm_o[wave][dl * 8 + j] = o[j];
  }
  if (lane == 0) { sm_m[wave] = m_run; sm_l[wave] = l_run; }
  __syncthreads();

  // merge the four wave summaries and write the partition's workspace entry
  float M = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
  const float M_use = (M == kNegInf) ? 0.f : M;
  float aw[4], L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) { aw[w] = fast_exp2(sm_m[w] - M_use); L += aw[w] * sm_l[w]; }
  const float inv = L == 0.f ? 0.f : 1.f / L;
  const int64_t prh = (int64_t)part * p.B * p.Nq * p.H + rh;
  if constexpr (!FUSED) {
    for (int d = tid; d < D; d += 256) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc = fmaf(aw[w], sm_o[w][d], acc);
      p.o_partial[prh * D + d] = acc * inv;
    }
    if (tid == 0) p.lse_partial[prh] = L == 0.f ? kNegInf : M_use + log2f(L);
  } else {
    // ---- publish this partition, then count it.  Only the first wave does this (the other
    //      three leave now and free their slots for other workgroups): it writes the entry with
    //      device-coherent stores (they bypass the per-XCD L2s, which are not coherent with one
    //      another), waits until those stores have completed, and takes the row-head's ticket
    //      with a device-coherent atomic.  The wave that draws the last ticket was therefore
    //      preceded by every other partition's completed stores, and reads them back with
    //      device-coherent loads.  No cache-wide write-back or invalidate is needed (an
    //      agent-scope release/acquire fence would do both, in every workgroup).
    if (wave != 0) return;
    for (int d = lane; d < D; d += 64) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc = fmaf(aw[w], sm_o[w][d], acc);
      put_ws<true>(p.o_partial + prh * D + d, acc * inv);
    }
    if (lane == 0) put_ws<true>(p.lse_partial + prh, L == 0.f ? kNegInf : M_use + log2f(L));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // keeps the stores before the ticket
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(p.tickets + rh * ATTN_TICKET_STRIDE_DEV, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    t = __builtin_amdgcn_readfirstlane(t);
    if (t != (uint32_t)p.P - 1u) return;
    // ---- last partition of this row-head: merge the P entries in this wave
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __shared__ float sc_tab[ATTN_P_MAX_DEV];
    const int64_t RH = (int64_t)p.B * p.Nq * p.H;
    // LSE phase: lane holds partitions lane + 64 j (P <= 256)
    float lsv[ATTN_P_MAX_DEV / 64];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < ATTN_P_MAX_DEV / 64; ++j) {
      const int pp = lane + 64 * j;
      lsv[j] = pp < p.P ? get_ws(p.lse_partial + (int64_t)pp * RH + rh) : kNegInf;
      mx = fmaxf(mx, lsv[j]);
    }
    mx = across_groups_max<1>(mx);
    float e = 0.f;
#pragma unroll
    for (int j = 0; j < ATTN_P_MAX_DEV / 64; ++j) e += (lsv[j] == kNegInf) ? 0.f : fast_exp2(lsv[j] - mx);
    e = group_sum<64>(e);
    const bool empty = (mx == kNegInf);
    const float Gl = empty ? kNegInf : log2f(e) + mx;
#pragma unroll
    for (int j = 0; j < ATTN_P_MAX_DEV / 64; ++j) {
      const int pp = lane + 64 * j;
      if (pp < p.P) sc_tab[pp] = (empty || lsv[j] == kNegInf) ? 0.f : fast_exp2(lsv[j] - Gl);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");   // the table is complete before it is read
    // weighted sum: lane covers d = lane + 64 i; eight partitions' entries are loaded before any
    // of them is folded, so the merge waits for ceil(P / 8) round trips to memory, not P
    constexpr int kBatch = 8;
    for (int d = lane; d < D; d += 64) {
      float acc = 0.f;
      const float* col = p.o_partial + rh * D + d;
      for (int pp0 = 0; pp0 < p.P; pp0 += kBatch) {
        float x[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          x[j] = pp0 + j < p.P ? get_ws(col + (int64_t)(pp0 + j) * RH * D) : 0.f;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const float sp = pp0 + j < p.P ? sc_tab[pp0 + j] : 0.f;
          acc = sp != 0.f ? fmaf(sp, x[j], acc) : acc;   // an empty partition adds nothing
        }
      }
      ((uint16_t*)p.out)[rh * D + d] = (uint16_t)(E::pack2(acc, 0.f) & 0xFFFFu);
    }
    if (lane == 0) {
      if (p.lse) p.lse[rh] = empty ? kNegInf : Gl * kLn2;
      __hip_atomic_store(p.tickets + rh * ATTN_TICKET_STRIDE_DEV, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
    }
  }
}

template <typename T, int D, bool FUSED>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)p.B * p.Nq * p.H * p.P));
  if (p.mask) hipLaunchKernelGGL((attn_decode_kernel<T, D, true, FUSED>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((attn_decode_kernel<T, D, false, FUSED>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, bool FUSED>
static hipError_t launch_decode_dtype(const DecodeParams& p, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_decode_t<T, 16, FUSED>(p, s);
    case 32: return launch_decode_t<T, 32, FUSED>(p, s);
    case 64: return launch_decode_t<T, 64, FUSED>(p, s);
    case 128: return launch_decode_t<T, 128, FUSED>(p, s);
    case 256: return launch_decode_t<T, 256, FUSED>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int dtype, int D, bool fused, hipStream_t s) {
  if (fused) return dtype == 0 ? launch_decode_dtype<bf16_t, true>(p, D, s) : launch_decode_dtype<f16_t, true>(p, D, s);
  return dtype == 0 ? launch_decode_dtype<bf16_t, false>(p, D, s) : launch_decode_dtype<f16_t, false>(p, D, s);
}

}  // namespace attn
