// attn_fwd.hip -- tiled attention forward on gfx950 matrix cores with the online-softmax
// recurrence.  Also the per-partition producer of the split-K workspace when Nq > 1.
//
// Method (triton-cuda-lab workshop "A3. Tiled attention with online normalization", sections
// "Keep three quantities for each query row" and "Masks that preserve the recurrence"; Tylo.jl
// "Streaming attention and online state", sections "Online statistics" and "Attention as a
// consumer"): per query keep the running maximum m, the FP32 denominator l and the FP32
// numerator a; for every key tile compute the scores, m' = max(m, rowmax), alpha = 2^(m - m'),
// p = 2^(s - m'), l = alpha*l + sum p, a = alpha*a + p V; finish with a / l.  Scores live in
// log2 units (logit * log2(e)), so every exponential is one v_exp_f32.
//
// Work decomposition (CDNA4 form of the pages' ownership rule that a row reduction must stay
// inside one wave): one workgroup of four waves per (query block of 128 rows, head, batch,
// partition); each wave owns 32 whole query rows and the block's full key range, so no
// cross-wave exchange is ever needed.
//
// Transposed products: the kernel computes S^T = K Q^T and O^T = V^T P^T.  In both
// accumulators a lane owns one query COLUMN, so the per-query state (m, l, alpha) is one scalar
// per lane and the score and output accumulators share it (Tylo "Online statistics": state and
// values must agree on the reduced ownership).  The K rows fed to the first product are
// permuted (pi below) so that the fp32 score registers of a lane, packed pairwise to bf16/fp16,
// ARE that lane's B operand of the second product: the accumulator-to-operand conversion needs
// no lane exchange (the CDNA4 counterpart of Tylo's "Same-lane conversion").
//
// Masking uses selects, never branches around the exponential (Tylo "Attention as a consumer"):
// the key tail and causal selects run only on tiles that need them, the byte mask on every
// tile when present.  Wholly future causal tiles are skipped (they would leave the state
// unchanged: workshop "Masks that preserve the recurrence").
#include "device.h"
#include "launch.h"

namespace attn {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;  // 128 query rows per workgroup

// Row permutation of a 32-key block inside the first product: A-operand row i holds key pi(i).
// With it, accumulator register r of lane l holds key 16*(r/8) + 8*(l/32) + (r%8), which is
// exactly the B-operand slot order of the second product for key step 2*mt + r/8.
__device__ __forceinline__ int key_perm(int i) {
  int b = i >> 3, h = (i >> 2) & 1;
  return ((b >> 1) << 4) + (h << 3) + ((b & 1) << 2) + (i & 3);
}

template <typename T, int D, int BN, bool MASK, bool SPLIT>
__global__ __launch_bounds__(256, (D >= 256 ? 1 : 2)) void attn_fwd_kernel(FwdParams p) {
  using E = elem<T>;
  constexpr int DP = D < 32 ? 32 : D;   // rows of O^T (padded to one 32-row MFMA tile)
  constexpr int KS = D + 8;             // LDS row stride of K (elements), 16 B of padding
  constexpr int VS = DP + 8;            // LDS row stride of V
  constexpr int KSTEPS = D / 16;        // k-steps of S^T = K Q^T
  constexpr int MT = BN / 32;           // 32-key blocks per tile
  constexpr int DT = DP / 32;           // 32-row tiles of O^T
  constexpr int PK = BN / 16;           // k-steps of O^T = V^T P^T
  constexpr int CH = D / 8;             // 16-byte chunks per K/V row
  constexpr int CHUNKS = BN * CH;       // chunks per K (and per V) tile
  constexpr int CPT = (CHUNKS + 255) / 256;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- block coordinates: h fastest, then b, then partition, then query block (longest first)
  int bid = blockIdx.x;
  const int h = bid % p.H; bid /= p.H;
  const int b = bid % p.B; bid /= p.B;
  const int part = bid % p.P; bid /= p.P;
  const int qb = p.causal ? (p.n_qblocks - 1 - bid) : bid;

  const int q_block0 = qb * kBlockM;
  const int q0 = q_block0 + wave * kRowsPerWave;   // first query row of this wave
  const int qi = q0 + (lane & 31);                 // query row (column of S^T) owned by this lane

  int kbeg = 0, kend = p.Nkv;
  if (SPLIT) {
    kbeg = part * p.chunk;
    kend = min(kbeg + p.chunk, p.Nkv);
  }
  if (p.causal) kend = min(kend, q_block0 + kBlockM);   // keys beyond the block's last row are future
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const int64_t row_stride = (int64_t)p.H * D;            // elements between consecutive tokens
  const uint16_t* qbase = (const uint16_t*)p.q + ((int64_t)b * p.Nq * p.H + h) * D;
  const uint16_t* kbase = (const uint16_t*)p.k + ((int64_t)b * p.Nkv * p.H + h) * D;
  const uint16_t* vbase = (const uint16_t*)p.v + ((int64_t)b * p.Nkv * p.H + h) * D;

  // D < 32: O^T rows D..31 read zero V columns (set once; staging never writes them).
  if constexpr (DP != D) {
    for (int i = tid; i < BN * (VS - D); i += 256) {
      int r = i / (VS - D), c = D + i % (VS - D);
      Vs[r * VS + c] = 0;
    }
  }

  // ---- Q^T as the B operand of S^T = K Q^T: lane holds Q[qi][16*ks + 8*(lane/32) .. +8]
  u32x4 qf[KSTEPS];
  {
    const bool ok = qi < p.Nq;
    const uint16_t* qrow = qbase + (int64_t)(ok ? qi : 0) * row_stride + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 v = ld16(qrow + 16 * ks);
      qf[ks] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }

  // ---- running state (one query per lane; replicated in lanes l and l^32)
  float m_run = kNegInf;   // running max of log2-unit scores
  float l_run = 0.f;       // this lane's partial denominator (its 16 keys of every 32)
  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};

  const float c = p.scale_log2;   // log2(e) / sqrt(D)

  // register staging of the next tile (prefetched while the current one is computed)
  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int t) {
    const int k0 = kbeg + t * BN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cidx = tid + i * 256;
      if (CHUNKS % 256 == 0 || cidx < CHUNKS) {
        const int r = cidx / CH, cc = cidx % CH;
        int key = k0 + r;
        key = key < p.Nkv ? key : p.Nkv - 1;   // rows past the end are masked; read a valid row
        kreg[i] = ld16(kbase + (int64_t)key * row_stride + cc * 8);
        vreg[i] = ld16(vbase + (int64_t)key * row_stride + cc * 8);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cidx = tid + i * 256;
      if (CHUNKS % 256 == 0 || cidx < CHUNKS) {
        const int r = cidx / CH, cc = cidx % CH;
        *reinterpret_cast<u32x4*>(&Ks[r * KS + cc * 8]) = kreg[i];
        *reinterpret_cast<u32x4*>(&Vs[r * VS + cc * 8]) = vreg[i];
      }
    }
  };

  const bool wave_has_rows = q0 < p.Nq;
  if (ntiles > 0) load_tile(0);

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = kbeg + t * BN;
    __syncthreads();          // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    // wave-uniform decisions for this tile
    const bool future = p.causal && (k0 > q0 + kRowsPerWave - 1);   // no key visible to any row
    if (!wave_has_rows || future) continue;
    const bool need_tail = (k0 + BN > kend);
    const bool need_causal = p.causal && (k0 + BN - 1 > q0);

    // ---- S^T = K Q^T  (MT blocks of 32 keys x 32 queries)
    f32x16 sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sacc[mt] = f32x16{};
      const uint16_t* krow = &Ks[(mt * 32 + key_perm(lane & 31)) * KS + 8 * (lane >> 5)];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 a = *reinterpret_cast<const u32x4*>(krow + 16 * ks);
        sacc[mt] = E::mfma32(a, qf[ks], sacc[mt]);
      }
    }

    // ---- masks (select to -inf).  Register r of block mt holds key
    //      k0 + 32*mt + 16*(r/8) + 8*(lane/32) + r%8 for query qi.
    const int kl = 8 * (lane >> 5);
    if (need_tail || need_causal) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * mt + 16 * (r >> 3) + kl + (r & 7);
          const bool vis = (key < kend) && (!p.causal || key <= qi);
          sacc[mt][r] = vis ? sacc[mt][r] : kNegInf;
        }
    }
    if constexpr (MASK) {
      const int qm = qi < p.Nq ? qi : p.Nq - 1;
      const uint8_t* mrow = p.mask + (int64_t)qm * p.Nkv;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int key0 = k0 + 32 * mt + 16 * hf + kl;   // 8 consecutive keys
          uint32_t lo = 0, hi = 0;
          if (p.mask_vec && key0 + 8 <= p.Nkv) {
            u32x2 w = *reinterpret_cast<const u32x2*>(mrow + key0);
            lo = w[0]; hi = w[1];
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int key = key0 + j;
              uint32_t byte = key < p.Nkv ? mrow[key] : 0u;
              if (j < 4) lo |= byte << (8 * j); else hi |= byte << (8 * (j - 4));
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t byte = (j < 4 ? (lo >> (8 * j)) : (hi >> (8 * (j - 4)))) & 0xFFu;
            const int r = 8 * hf + j;
            sacc[mt][r] = byte ? sacc[mt][r] : kNegInf;
          }
        }
    }

    // ---- online softmax update (one query per lane)
    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    mx = xor32_max(mx);                              // the other 16 keys of each block
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;   // all-masked so far: no -inf - -inf
    const float alpha = fast_exp2(m_run - m_use);           // 0 from the empty state
    m_run = m_new;

    float psum = 0.f;
    u32x4 pf[PK];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = fast_exp2(fmaf(sacc[mt][8 * hf + j], c, -m_use));   // masked: 2^-inf = 0
          psum += pv[j];
        }
        pf[2 * mt + hf] = u32x4{E::pack2(pv[0], pv[1]), E::pack2(pv[2], pv[3]),
                                E::pack2(pv[4], pv[5]), E::pack2(pv[6], pv[7])};
      }
    l_run = alpha * l_run + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

    // ---- O^T += V^T P^T.  A operand (V^T, 32 d-rows x 16 keys) through transposing LDS reads:
    //      16-lane group g covers d = 32*dt + 16*(g%2) .. +16 and keys 16*kk + 8*(g/2) + {0..3},
    //      {4..7}; lane 4*j + tq of the group addresses key row (.. + j), d chunk 4*tq.
    {
      const int g = lane >> 4, li = lane & 15;
      const int jrow = li >> 2, tq = li & 3;
#pragma unroll
      for (int kk = 0; kk < PK; ++kk) {
        const int krow = 16 * kk + 8 * (g >> 1) + jrow;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int dcol = 32 * dt + 16 * (g & 1) + 4 * tq;
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&Vs[krow * VS + dcol]);
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&Vs[(krow + 4) * VS + dcol]);
          u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          u32x4 a = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
          oacc[dt] = E::mfma32(a, pf[kk], oacc[dt]);
        }
      }
    }
  }

  // ---- epilogue: finish the denominator over the lane pair, normalise, store
  const float l_all = xor32_sum(l_run);
  const float inv = l_all == 0.f ? 0.f : 1.f / l_all;
  const bool row_ok = qi < p.Nq;
  const int64_t rh = ((int64_t)b * p.Nq + qi) * p.H + h;   // row-head index

  if constexpr (!SPLIT) {
    if (row_ok) {
      uint16_t* orow = (uint16_t*)p.out + rh * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int d0 = 32 * dt + 8 * rb + 4 * (lane >> 5);
          if (d0 < D) {
            u32x2 w = u32x2{E::pack2(oacc[dt][4 * rb + 0] * inv, oacc[dt][4 * rb + 1] * inv),
                            E::pack2(oacc[dt][4 * rb + 2] * inv, oacc[dt][4 * rb + 3] * inv)};
            *reinterpret_cast<u32x2*>(orow + d0) = w;
          }
        }
      if (p.lse && lane < 32)
        p.lse[rh] = l_all == 0.f ? kNegInf : (m_run + log2f(l_all)) * kLn2;
    }
  } else {
    if (row_ok) {
      const int64_t prh = (int64_t)part * p.B * p.Nq * p.H + rh;
      float* orow = p.o_partial + prh * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int d0 = 32 * dt + 8 * rb + 4 * (lane >> 5);
          if (d0 < D) {
            f32x4 w = f32x4{oacc[dt][4 * rb + 0] * inv, oacc[dt][4 * rb + 1] * inv,
                            oacc[dt][4 * rb + 2] * inv, oacc[dt][4 * rb + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + d0) = w;
          }
        }
      if (lane < 32) p.lse_partial[prh] = l_all == 0.f ? kNegInf : m_run + log2f(l_all);
    }
  }
}

// ---- host-side dispatch -------------------------------------------------------------------
template <typename T, int D, int BN, bool MASK, bool SPLIT>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)p.n_qblocks * p.H * p.B * p.P));
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, MASK, SPLIT>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D, int BN>
static hipError_t launch_fwd_mask(const FwdParams& p, bool split, hipStream_t s) {
  const bool mask = p.mask != nullptr;
  if (split) return mask ? launch_fwd_t<T, D, BN, true, true>(p, s) : launch_fwd_t<T, D, BN, false, true>(p, s);
  return mask ? launch_fwd_t<T, D, BN, true, false>(p, s) : launch_fwd_t<T, D, BN, false, false>(p, s);
}

template <typename T>
static hipError_t launch_fwd_dtype(const FwdParams& p, int D, int BN, bool split, hipStream_t s) {
  switch (D) {
    case 16: return BN == 32 ? launch_fwd_mask<T, 16, 32>(p, split, s) : launch_fwd_mask<T, 16, 64>(p, split, s);
    case 32: return BN == 32 ? launch_fwd_mask<T, 32, 32>(p, split, s) : launch_fwd_mask<T, 32, 64>(p, split, s);
    case 64: return BN == 32 ? launch_fwd_mask<T, 64, 32>(p, split, s) : launch_fwd_mask<T, 64, 64>(p, split, s);
    case 128: return launch_fwd_mask<T, 128, 64>(p, split, s);
    case 256: return launch_fwd_mask<T, 256, 64>(p, split, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int BN, bool split, hipStream_t s) {
  return dtype == 0 ? launch_fwd_dtype<bf16_t>(p, D, BN, split, s) : launch_fwd_dtype<f16_t>(p, D, BN, split, s);
}

int fwd_block_m() { return kBlockM; }

}  // namespace attn
