// attn_fwd_kernel.h -- the tiled attention forward kernel (gfx950 matrix cores, online-softmax
// recurrence) and its launch templates, shared by attn_fwd.hip (D <= 128, the FP8-V form) and
// attn_fwd_d256.hip (D = 256, built with its own scheduling flags).  Also the per-partition
// producer of the split-K workspace when Nq > 1.
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
// inside one wave): one workgroup of WAVES waves per (query block of 32*WAVES rows, head, batch,
// partition); each wave owns 32 whole query rows and the block's full key range, so no
// cross-wave exchange is ever needed.  The waves share the K and V tiles, which are staged
// into LDS by direct global-to-LDS loads, two or three stages deep, one barrier per tile.
//
// Transposed products: the kernel computes S^T = K Q^T and O^T = V^T P^T.  In both
// accumulators a lane owns one query COLUMN, so the per-query state (m, l, alpha) is one scalar
// per lane and the score and output accumulators share it (Tylo "Online statistics": a summary
// serves only values distributed over the lanes the same way it is).  The K rows fed to the first product are
// permuted (pi below) so that the fp32 score registers of a lane, packed pairwise to bf16/fp16,
// ARE that lane's B operand of the second product: the accumulator-to-operand conversion needs
// no lane exchange (the CDNA4 counterpart of Tylo's "Same-lane conversion").
//
// Masking uses selects, never branches around the exponential (Tylo "Attention as a consumer"):
// the key tail and causal selects run only on tiles that need them, the byte mask on every
// tile when present; the byte mask's tile (the block's rows x the tile's keys) is staged into
// LDS with the K and V tiles when its rows are 16-byte aligned, and read from global memory
// otherwise.  Wholly future causal tiles are skipped (they would leave the state
// unchanged: workshop "Masks that preserve the recurrence").
#pragma once
#include "device.h"
#include "launch.h"

#include <type_traits>

namespace attn {

constexpr int kRowsPerWave = 32;               // query rows (accumulator columns) per wave
constexpr int kMinBlockM = 4 * kRowsPerWave;   // smallest query block (four waves)

// Lazy rescale threshold (log2 units): the reference maximum m is raised only when a weight
// against the current reference could exceed 2^TAU, so weights stay <= 2^TAU and the O rescale
// is skipped on almost every block.  O / l and m + log2(l) do not depend on which reference is
// used.
constexpr float kTau = 8.0f;
constexpr float kTauPow = 256.0f;   // 2^TAU

// Source of the byte mask, fixed per instantiation: a run-time choice inside the tile body would
// split it into basic blocks, and the scheduler interleaves matrix and vector instructions only
// inside one.
constexpr int kMaskNone = 0;     // no byte mask
constexpr int kMaskLds = 1;      // mask tiles staged into LDS with K and V (16-byte aligned rows)
constexpr int kMaskGlobal = 2;   // mask bytes read from global memory (8 at a time when aligned)
constexpr int kMaskBits = 3;     // packed mask (attn_mask_pack): one word per lane per 64 keys,
                                 // loaded a tile ahead into a register (unsplit launches)

// LDS chunk swizzles (16-byte chunk index XOR, per key row).
template <int SWZ>
__device__ __forceinline__ int k_swz(int row) { return row & SWZ; }
template <int RPB, int BITS>
__device__ __forceinline__ int v_swz(int row) { return BITS ? 4 * ((row / RPB) & BITS) : 0; }

template <int S> using stage_t = std::integral_constant<int, S>;

// s where bit b of w is set, else -inf: the bit sign-extended to a full mask (one bit-field
// extract), then one bit-field select between s and -inf.
__device__ __forceinline__ float keep_if_bit(uint32_t w, int b, float s) {
  const uint32_t m = (uint32_t)((int32_t)(w << (31 - b)) >> 31);
  return __uint_as_float((__float_as_uint(s) & m) | (0xff800000u & ~m));
}

// s where byte B of w is nonzero, else -inf: one compare of the byte against 0 (SDWA operand
// select) into a lane mask, and one select.  Only the compare is written out (the compiler
// extracts most bytes with a separate AND or shift first); the select stays compiler-generated
// because s is usually a matrix-core result, whose read-after-write wait states the compiler
// inserts for its own instructions but not for inline asm.
template <int B>
__device__ __forceinline__ float keep_if_byte(uint32_t w, float s) {
  static_assert(B >= 0 && B < 4, "byte index");
  uint64_t m;
#define ATTN_BYTE_NZ(SEL) \
  asm("v_cmp_ne_u32_sdwa %0, %1, %2 src0_sel:" SEL " src1_sel:DWORD" : "=s"(m) : "v"(w), "v"(0u))
  if constexpr (B == 0) ATTN_BYTE_NZ("BYTE_0");
  else if constexpr (B == 1) ATTN_BYTE_NZ("BYTE_1");
  else if constexpr (B == 2) ATTN_BYTE_NZ("BYTE_2");
  else ATTN_BYTE_NZ("BYTE_3");
#undef ATTN_BYTE_NZ
  return __builtin_amdgcn_inverse_ballot_w64(m) ? s : -__builtin_inff();
}

// WAVES waves of 32 query rows each; BN keys per tile.
// V8: 0 = V in T; 1 / 2 = V in E4M3 / E5M2 (one byte per element) and the second product on the
// FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4, one 64-key tile per instruction) with P rounded
// to E4M3.
// PAIR (causal launches): a workgroup runs query blocks n-1-i and then i of one unit.
template <typename T, int D, int BN, int MASK, bool SPLIT, int WAVES, int NSTAGES, int V8 = 0, bool PAIR = false>
__global__ __launch_bounds__(64 * WAVES, (WAVES >= 8 || D >= 256) ? 1 : 2) void attn_fwd_kernel(FwdParams p) {
  using E = elem<T>;
  constexpr int kBlockM = WAVES * kRowsPerWave;
  constexpr int DP = D < 32 ? 32 : D;   // rows of O^T (padded to one 32-row MFMA tile)
  constexpr int RB = D * 2;             // bytes per K / V row in LDS (unpadded)
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int SWZ = CH < 16 ? CH - 1 : 15;   // K chunk index XOR (row & SWZ): conflict-free b128 reads
  // V chunk XOR: the four key rows one transposing read touches must fall on distinct banks
  constexpr int RPB = RB >= 256 ? 1 : 256 / RB;            // key rows per 256-byte bank line
  constexpr int VSWZ_BITS = CH >= 16 ? 3 : (CH >= 8 ? 1 : 0);
  constexpr int TILE = BN * RB;         // bytes of one K (or V) tile
  constexpr int NT = TILE / 1024;       // 1 KiB wave-instructions per tile per tensor
  constexpr int RPI = 1024 / RB;        // rows covered by one wave-instruction
  constexpr int KSTEPS = D / 16;        // k-steps of S^T = K Q^T
  constexpr int MT = BN / 32;           // 32-key blocks per tile
  constexpr int DT = DP / 32;           // 32-row tiles of O^T
  // Mask tiles (MASK): the block's kBlockM query rows x BN key bytes, staged through LDS like K
  // and V.  Row r's 16-byte chunk c sits at position c ^ msw(r) of the row, so the 32 rows one
  // wave reads with a single instruction spread over the banks.
  constexpr int MTILE = MASK == kMaskLds ? kBlockM * BN : 0;
  constexpr int M_CPR = BN / 16;                  // 16-byte chunks per mask row
  constexpr int M_RPI = 64 / M_CPR;               // mask rows per wave-instruction
  constexpr int M_RPL = 256 / BN;                 // mask rows per 256-byte bank line
  constexpr int MPW = MTILE / (1024 * WAVES);      // mask wave-instructions per wave per tile
  static_assert(MTILE % (1024 * WAVES) == 0, "whole mask wave-instructions per wave");
  static_assert((WAVES * M_RPI / M_RPL) % M_CPR == 0, "mask swizzle independent of the instruction");
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves per workgroup");
  static_assert(TILE % 1024 == 0, "tile must be a whole number of 1 KiB wave loads");
  // V tiles: 2 bytes per element, or 1 with V8.  V8 rows (D bytes, 8 chunks) are swizzled by
  // chunk ^ (2 * ((row / 2) % 4)): the 8 rows x 2 chunks that one half-wave of a byte-transposing
  // read touches then cover the 64 banks exactly once.
  static_assert(!V8 || (D == 128 && (BN == 64 || BN == 128) && !SPLIT), "the FP8 second product is built for D = 128, 64- or 128-key tiles");
  static_assert(MASK != kMaskBits || BN <= 64, "a packed-mask word covers 64 keys");
  static_assert(MASK != kMaskBits || !SPLIT, "packed masks assume key tiles aligned to 64 keys");
  constexpr int RBV = V8 ? D : RB;      // bytes per V row in LDS
  constexpr int TILEV = BN * RBV;
  constexpr int NTV = TILEV / 1024;
  constexpr int RPIV = 1024 / RBV;
  constexpr int CHV = RBV / 16;
  constexpr int PER_WAVE_V8 = (NTV + WAVES - 1) / WAVES;
  // LDS stages: tiles are loaded NSTAGE-1 ahead.  Three stages where one workgroup owns the CU
  // (eight waves), two otherwise.
  constexpr int NSTAGE = NSTAGES;
  static_assert(NSTAGE == 2 || NSTAGE == 3, "two or three LDS stages");
  // LDS: [K stages | V stages].  Every operand read is a per-lane base plus a compile-time offset
  // (block, key step, stage), which must fit the 16-bit DS offset.
  constexpr int K_OFS = 0, V_OFS = NSTAGE * TILE;
  constexpr int KS_PER = KSTEPS < (SWZ + 1) / 2 ? KSTEPS : (SWZ + 1) / 2;   // key steps per K swizzle group
  constexpr int DT_PER = DT < 4 ? DT : 4;                                  // row tiles per V swizzle group
  static_assert(VSWZ_BITS != 1 || DT <= 2, "V swizzle groups of two row tiles");
  static_assert((NSTAGE - 1) * TILE + (MT - 1) * 32 * RB + 16 * (SWZ + 1) * ((KSTEPS - 1) / KS_PER) < 65536,
                "K read offsets exceed the DS immediate");
  static_assert((NSTAGE - 1) * TILEV + (BN - 1) * RBV + 64 * DT_PER * ((DT - 1) / DT_PER) < 65536,
                "V read offsets exceed the DS immediate");

  constexpr int M_OFS = NSTAGE * (TILE + TILEV);
  static_assert(M_OFS + NSTAGE * MTILE <= 160 * 1024, "LDS budget of one workgroup");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[M_OFS + NSTAGE * MTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- block coordinates.  Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8),
  //      so the linear order is remapped to give each XCD a contiguous run of blocks: the query
  //      blocks of one (head, batch) then run together on one XCD and share its L2 for K and V.
  //      Causal blocks differ in length (query block i visits i+1 key blocks).  With PAIR a
  //      workgroup runs blocks n-1-i and i (n+1 key blocks in all), so every workgroup is equally
  //      long and a CU is refilled as soon as its workgroup ends (workgroups that end at different
  //      times leave CUs idle for microseconds between them); otherwise blocks are issued longest
  //      first.  Both are issued over PAIRS of heads: with one head at a time the long blocks of
  //      the last heads would start late and finish after everything else.
  int bid = blockIdx.x;
  if (gridDim.x % 8 == 0) bid = (bid % 8) * (gridDim.x / 8) + bid / 8;
  const int n_heads = p.H * p.B * p.P;                 // (head, batch, partition) units
  const int per_unit = PAIR ? (p.n_qblocks + 1) / 2 : p.n_qblocks;   // workgroups per unit
  int hl, qb_idx;
  if (p.causal && n_heads % 2 == 0) {
    const int hh = bid & 1;
    bid >>= 1;
    qb_idx = bid % per_unit;
    hl = 2 * (bid / per_unit) + hh;
  } else {
    qb_idx = bid % per_unit;
    hl = bid / per_unit;
  }
  // the (first) block: causal ones longest first
  const int qb_first = p.causal ? (p.n_qblocks - 1 - qb_idx) : qb_idx;

  // With PAIR, the second block's Q rows are loaded into qn at the end of the first block's tile
  // loop: their latency then overlaps the first block's epilogue and the barrier between the
  // blocks (where the waves whose rows left the causal diagonal first wait for the others).
  u32x4 qn[PAIR ? KSTEPS : 1];
  auto load_q = [&](int qb, u32x4* dst) __attribute__((always_inline)) {
    const int h = hl % p.H, b = (hl / p.H) % p.B;
    const int qi = qb * kBlockM + wave * kRowsPerWave + (lane & 31);
    const bool ok = qi < p.Nq;
    const uint16_t* qrow = (const uint16_t*)p.q + ((int64_t)b * p.Nq * p.H + h) * D + (int64_t)(ok ? qi : 0) * ((int64_t)p.H * D) + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 v = ld16(qrow + 16 * ks);
      dst[ks] = ok ? v : u32x4{0, 0, 0, 0};
    }
  };
  // blk_c: 0 = a single block, 1 = the first block of a pair, 2 = the second
  auto run_block = [&](const int qb, auto blk_c) __attribute__((always_inline)) {
    constexpr int BLK = decltype(blk_c)::value;
  const int h = hl % p.H;
  const int b = (hl / p.H) % p.B;
  const int part = hl / (p.H * p.B);

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

  // ---- packed mask: word ((q0 / 32) * n_kgroups + key group) * 64 + lane holds this lane's
  //      scores of 64 keys, bit 16 mt + r for register r of 32-key block mt.  The word of tile
  //      t + 1 is loaded while tile t runs (a 32-key tile takes its half of the word).
  constexpr bool use_bits = MASK == kMaskBits;
  const uint32_t* mbits_lane = use_bits ? p.mask_bits + (int64_t)(q0 >> 5) * p.n_kgroups * 64 + lane : nullptr;
  auto load_bits = [&](int t) -> uint32_t {
    const int kt = t * BN;
    const uint32_t w = mbits_lane[(int64_t)(kt >> 6) * 64];
    return BN == 32 ? (w >> (16 * ((kt >> 5) & 1))) : w;
  };
  uint32_t mbits_next = 0;
  if constexpr (use_bits)
    if (q0 < p.Nq && ntiles > 0) mbits_next = load_bits(0);

  const int64_t row_stride = (int64_t)p.H * D;            // elements between consecutive tokens
  const uint16_t* qbase = (const uint16_t*)p.q + ((int64_t)b * p.Nq * p.H + h) * D;
  const uint16_t* kbase = (const uint16_t*)p.k + ((int64_t)b * p.Nkv * p.H + h) * D;
  const uint16_t* vbase = (const uint16_t*)p.v + ((int64_t)b * p.Nkv * p.H + h) * D;
  const uint8_t* vbase8 = (const uint8_t*)p.v + ((int64_t)b * p.Nkv * p.H + h) * D;   // V8

  // ---- direct global -> LDS staging (buffer_load ... lds).  Wave-instruction j of a tile fills
  //      LDS bytes [1024 j, 1024 j + 1024): lane l lands at row j*RPI + l/CH, physical chunk
  //      l%CH, which holds logical chunk (l%CH) ^ swizzle(row) of that key row.  The per-lane
  //      byte offsets inside a tile are fixed; each tile only moves the scalar base.
  constexpr int PER_WAVE = (NT + WAVES - 1) / WAVES;
  // Row of instruction jj = (jj*WAVES + wave)*RPI + lane/CH.  When WAVES*RPI is a multiple of 16
  // (D <= 128) neither swizzle depends on jj, so one per-lane offset serves every instruction and
  // the jj part goes into the scalar offset.
  constexpr bool ONE_OFS = (WAVES * RPI) % 16 == 0;
  const int ld_row_in = lane / CH;
  const int ld_pc = lane % CH;
  const int row0 = wave * RPI + ld_row_in;
  const uint32_t kvo0 = (uint32_t)(((int64_t)row0 * row_stride + 8 * (ld_pc ^ k_swz<SWZ>(row0))) * 2);
  const uint32_t vvo0 = (uint32_t)(((int64_t)row0 * row_stride + 8 * (ld_pc ^ v_swz<RPB, VSWZ_BITS>(row0))) * 2);
  const uint32_t jj_bytes = (uint32_t)((int64_t)WAVES * RPI * row_stride * 2);   // scalar step per jj
  const uint32_t tile_bytes = (uint32_t)((int64_t)BN * row_stride * 2);
  // s_waitcnt immediate for "vmcnt <= the loads of one tile" (gfx9 encoding: vmcnt in bits 3:0
  // and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima, i.e. not waited for)
  constexpr int kTileLoads = PER_WAVE + (V8 ? PER_WAVE_V8 : PER_WAVE);
  static_assert(NSTAGE == 2 || NT % WAVES == 0, "three stages need the same load count in every wave");
  static_assert(NSTAGE == 2 || !V8 || NTV % WAVES == 0, "three stages need the same load count in every wave");
  constexpr int kWaitAllButOneTile = (kTileLoads & 15) | ((kTileLoads >> 4) << 14) | (7 << 4) | (15 << 8);
  constexpr int kTileLoadsM = kTileLoads + MPW;   // with the mask tile
  constexpr int kWaitAllButOneTileM = (kTileLoadsM & 15) | ((kTileLoadsM >> 4) << 14) | (7 << 4) | (15 << 8);
  // mask staging: lane offsets (row in the offset register, which the buffer bound checks: rows
  // at or past Nq, and bytes past the end of the mask, read as 0)
  constexpr bool use_lds_mask = MASK == kMaskLds;
  auto msw = [](int r) { return (r / M_RPL) % M_CPR; };
  const int mrow0 = wave * M_RPI + lane / M_CPR;
  const uint32_t mo0 = (uint32_t)mrow0 * (uint32_t)p.Nkv + 16u * (uint32_t)((lane % M_CPR) ^ msw(mrow0));
  const uint32_t m_step = (uint32_t)(WAVES * M_RPI) * (uint32_t)p.Nkv;
  // the LDS destination goes to M0, which must be provably wave-uniform
  const int wave_lds = __builtin_amdgcn_readfirstlane(wave * 1024);
  auto issue_tile = [&](int t, int stage) {
    const int k0 = kbeg + t * BN;
    uint8_t* kdst = lds + K_OFS + stage * TILE + wave_lds;
    uint8_t* vdst = lds + V_OFS + stage * TILEV + wave_lds;
    __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)k0 * row_stride), 0, tile_bytes, 0x00020000);
    __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)k0 * row_stride), 0, tile_bytes, 0x00020000);
    if (k0 + BN <= p.Nkv) {
#pragma unroll
      for (int jj = 0; jj < PER_WAVE; ++jj) {
        const int j = jj * WAVES + wave;
        if (NT % WAVES != 0 && j >= NT) break;
        uint32_t ko = kvo0, vo = vvo0, so = jj * jj_bytes;
        if constexpr (!ONE_OFS) {   // the swizzles depend on the instruction: per-lane offsets
          const int row = j * RPI + ld_row_in;
          ko = (uint32_t)(((int64_t)row * row_stride + 8 * (ld_pc ^ k_swz<SWZ>(row))) * 2);
          vo = (uint32_t)(((int64_t)row * row_stride + 8 * (ld_pc ^ v_swz<RPB, VSWZ_BITS>(row))) * 2);
          so = 0;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kdst + jj * WAVES * 1024), 16, ko, so, 0, 0);
        if constexpr (!V8)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vdst + jj * WAVES * 1024), 16, vo, so, 0, 0);
      }
    } else {   // last tile: rows past the end are masked; read the last valid row instead
#pragma unroll
      for (int jj = 0; jj < PER_WAVE; ++jj) {
        const int j = jj * WAVES + wave;
        if (NT % WAVES != 0 && j >= NT) break;
        const int row = j * RPI + ld_row_in;
        const int rr = (k0 + row < p.Nkv ? k0 + row : p.Nkv - 1) - k0;
        const uint32_t ko = (uint32_t)(((int64_t)rr * row_stride + 8 * (ld_pc ^ k_swz<SWZ>(row))) * 2);
        const uint32_t vo = (uint32_t)(((int64_t)rr * row_stride + 8 * (ld_pc ^ v_swz<RPB, VSWZ_BITS>(row))) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kdst + jj * WAVES * 1024), 16, ko, 0, 0, 0);
        if constexpr (!V8)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vdst + jj * WAVES * 1024), 16, vo, 0, 0, 0);
      }
    }
    if constexpr (V8) {
      // byte rows of the E4M3 V tile: instruction jj of this wave covers rows
      // (jj*WAVES + wave)*RPIV + lane/CHV, physical chunk lane%CHV holding logical chunk
      // (lane%CHV) ^ (2 * ((row / 2) % 4)); rows past the key length read the last valid row
      const uint32_t v8_bytes = (uint32_t)((int64_t)BN * row_stride);
      __amdgpu_buffer_rsrc_t rv8 = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase8 + (int64_t)k0 * row_stride), 0, v8_bytes, 0x00020000);
#pragma unroll
      for (int jj = 0; jj < PER_WAVE_V8; ++jj) {
        const int j = jj * WAVES + wave;
        if (NTV % WAVES != 0 && j >= NTV) break;
        const int row = j * RPIV + lane / CHV;
        const int rr = (k0 + row < p.Nkv ? k0 + row : p.Nkv - 1) - k0;
        const uint32_t vo8 = (uint32_t)((int64_t)rr * row_stride + 16 * ((lane % CHV) ^ (2 * ((row >> 1) & 3))));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv8, (__attribute__((address_space(3))) void*)(vdst + jj * WAVES * 1024), 16, vo8, 0, 0, 0);
      }
    }
    if constexpr (use_lds_mask) {
      uint8_t* mdst = lds + M_OFS + stage * MTILE + wave_lds;
      const int64_t mbase = (int64_t)q_block0 * p.Nkv + k0;
      const uint32_t mbytes = (uint32_t)((int64_t)p.Nq * p.Nkv - mbase);   // to the end of the mask
      __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc((void*)(p.mask + mbase), 0, mbytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < MPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (__attribute__((address_space(3))) void*)(mdst + i * WAVES * 1024), 16, mo0 + i * m_step, 0, 0, 0);
    }
  };

  // ---- Q^T as the B operand of S^T = K Q^T: lane holds Q[qi][16*ks + 8*(lane/32) .. +8]
  u32x4 qf[KSTEPS];
  if constexpr (BLK == 2) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = qn[ks];
  } else {
    const bool ok = qi < p.Nq;
    const uint16_t* qrow = qbase + (int64_t)(ok ? qi : 0) * row_stride + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 v = ld16(qrow + 16 * ks);
      qf[ks] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }

  // ---- running state (one query per lane; replicated in lanes l and l^32)
  float m_run = kNegInf;   // reference maximum of log2-unit scores
  float l_run = 0.f;       // this lane's partial denominator (its 16 keys of every 32)
  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};

  const float c = p.scale_log2;   // log2(e) / sqrt(D)
  const bool wave_has_rows = q0 < p.Nq;
  const int kl = 8 * (lane >> 5);

  // ---- per-lane LDS byte addresses of the operand reads.  K operand (block mt, key step ks):
  //      row mt*32 + pi(lane%32), logical chunk 2*ks + lane/32, XOR the row swizzle (equal for
  //      every block since SWZ < 32).  V^T operand (block mt, key step k2, row tile dt) by
  //      transposing reads: 16-lane group g covers d = 32*dt + 16*(g%2) .. +16 and keys
  //      16*(2*mt + k2) + 8*(g/2) + {0..3}, {4..7}; lane 4*j + tq of the group addresses key row
  //      (.. + j), d chunk 4*tq.  Only the parts that depend on the lane are kept here; block,
  //      key step and stage are compile-time offsets.
  //      The chunk swizzles only permute chunks inside aligned groups of SWZ + 1 (K) and of 16
  //      (V, 4 row tiles), so one base per key step (row tile) of the first group serves the
  //      later groups with an immediate offset (D = 256 needs 8 + 4 fewer address registers).
  const uint8_t* kaddr[KS_PER];
  {
    const int krow = key_perm(lane & 31);
    const int ksw = k_swz<SWZ>(krow);
#pragma unroll
    for (int ks = 0; ks < KS_PER; ++ks)
      kaddr[ks] = lds + K_OFS + krow * RB + 16 * ((2 * ks + (lane >> 5)) ^ ksw);
  }
  // mask bytes of this lane's query row: chunk c (keys 16c .. 16c+15 of the tile), half kl
  const uint8_t* maddr[use_lds_mask ? M_CPR : 1];
  if constexpr (use_lds_mask) {
    const int rl = wave * kRowsPerWave + (lane & 31);
#pragma unroll
    for (int c = 0; c < M_CPR; ++c) maddr[c] = lds + M_OFS + rl * BN + 16 * (c ^ msw(rl)) + kl;
  }
  // V8: A operand of the FP8 second product (V^T: 32 rows of d x 64 keys) by byte-transposing
  // reads (ds_read_b64_tr_b8).  Per 16-lane group G, lane i receives byte (i % 16) % 8 of the
  // 8-byte chunks addressed by lanes 16 G + 2 j + (i % 16) / 8, j = 0..7 (measured on gfx950).
  // Operand byte 8 c + e of lane l must be V[16 c + 8 (l / 32) + e][32 dt + l % 32] (the key order
  // of the packed P bytes), so lane P addresses key row 16 c + 8 (G / 2) + (P % 16) / 2 at byte
  // 32 dt + 16 (G % 2) + 8 (P % 2); the row swizzle does not depend on c (rows move by 16 c).
  const uint8_t* vaddr8[V8 ? DT : 1];
  if constexpr (V8) {
    const int G = lane >> 4, pp = lane & 15;
    const int row = 8 * (G >> 1) + (pp >> 1);
    const int sw = 2 * ((row >> 1) & 3);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vaddr8[dt] = lds + V_OFS + row * D + 16 * ((2 * dt + (G & 1)) ^ sw) + 8 * (pp & 1);
  }
  const uint8_t* vaddr[DT_PER];
  const int g = lane >> 4, li = lane & 15;
  const bool dpad = (D < 32) && ((g & 1) != 0);    // O^T rows D..31 for D = 16: zero operand
  {
    const int jrow = li >> 2, tq = li & 3;
    const int vrow = 8 * (g >> 1) + jrow;          // the swizzle depends on the key row only through this
#pragma unroll
    for (int dt = 0; dt < DT_PER; ++dt) {
      const int d = 32 * dt + 16 * (g & 1) + 4 * tq;
      const int cidx = (d / 8) % CH;
      vaddr[dt] = lds + V_OFS + vrow * RB + 16 * (cidx ^ v_swz<RPB, VSWZ_BITS>(vrow)) + 8 * (tq & 1);
    }
  }

  // pins a value at this point: the weight sum depends on every exponential of the block, so
  // the common path stays ahead of the rare-branch test instead of being sunk into it
#if defined(__HIP_DEVICE_COMPILE__)
#define ATTN_PIN(x) asm volatile("" : "+v"(x))
#else
#define ATTN_PIN(x) (void)(x)   // the host pass only emits launch stubs
#endif

  // ---- one key tile: wait for it, start the next tile's loads, update the state
  auto do_tile = [&](const int t, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const int k0 = kbeg + t * BN;
    // tile t resident for every wave (its LDS-DMA loads are counted by vmcnt, which the
    // barrier's own fence does not wait for; with three stages the loads of tile t+1, issued
    // after it, may stay in flight); every wave done with tile t-1, whose stage is refilled next
    if (NSTAGE == 3 && t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(use_lds_mask ? kWaitAllButOneTileM : kWaitAllButOneTile);
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    uint32_t mw = 0;   // packed mask word of this tile
    if constexpr (use_bits) {
      // issued before the next stage's loads, so that the count-based wait at the start of tile
      // t + 1 (all but that stage's loads) covers it
      mw = mbits_next;
      if (t + 1 < ntiles && q0 < p.Nq && !(p.causal && k0 + BN > q0 + kRowsPerWave - 1)) mbits_next = load_bits(t + 1);
    }
    if (t + NSTAGE - 1 < ntiles) issue_tile(t + NSTAGE - 1, (S + NSTAGE - 1) % NSTAGE);

    // wave-uniform decisions for this tile
    const bool future = p.causal && (k0 > q0 + kRowsPerWave - 1);   // no key visible to any row
    if (!wave_has_rows || future) return;
    const bool need_tail = (k0 + BN > kend);
    const bool need_causal = p.causal && (k0 + BN - 1 > q0);

    auto read_k = [&](int mt, u32x4 (&kf)[KSTEPS]) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        kf[ks] = *reinterpret_cast<const u32x4*>(kaddr[ks % KS_PER] + S * TILE + mt * 32 * RB + 16 * (SWZ + 1) * (ks / KS_PER));
    };
    auto qk = [&](const u32x4 (&kf)[KSTEPS]) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) acc = E::mfma32(kf[ks], qf[ks], acc);
      return acc;
    };
    auto read_v = [&](int mt, u32x4 (&va)[2][DT]) {
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint8_t* a0 = vaddr[dt % DT_PER] + S * TILEV + 16 * (2 * mt + k2) * RB + 64 * DT_PER * (dt / DT_PER);
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 4 * RB));
          u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          va[k2][dt] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
          if (dpad) va[k2][dt] = u32x4{0, 0, 0, 0};
        }
    };
    auto pv = [&](const u32x4 (&va)[2][DT], const u32x4 (&pb)[2]) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = E::mfma32(va[k2][dt], pb[k2], oacc[dt]);
    };
    // Masks (select to -inf).  Register r of block mt holds key
    // k0 + 32*mt + 16*(r/8) + 8*(lane/32) + r%8 for query qi.  mask_block returns whether any of
    // the lane's 16 keys stays visible (for the rescale test's "no reference yet" clause).
    // The byte-mask words of block mt, keys 16*hf .. +8 (lo: bytes 0-3, hi: 4-7):
    auto mask_words = [&](int mt, int hf, uint32_t& lo, uint32_t& hi) {
      const int key0 = k0 + 32 * mt + 16 * hf + kl;   // 8 consecutive keys
      lo = 0; hi = 0;
      if constexpr (MASK == kMaskLds) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(maddr[2 * mt + hf] + S * MTILE);
        lo = w[0]; hi = w[1];
      } else {
        const int qm = qi < p.Nq ? qi : p.Nq - 1;
        const uint8_t* mrow = p.mask + (int64_t)qm * p.Nkv;
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
      }
    };
    auto mask_block = [&](int mt, f32x16& sa, auto masked_c) {
      constexpr bool IDX = decltype(masked_c)::value;
      if constexpr (!IDX && MASK == kMaskNone) {
        return true;
      } else if constexpr (!IDX && MASK == kMaskBits) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[r] = keep_if_bit(mw, 16 * mt + r, sa[r]);
        return ((mw >> (16 * mt)) & 0xffffu) != 0u;
      } else if constexpr (!IDX) {
        // byte mask only (no tail or causal test on this tile): two instructions per score
        uint32_t w[4];
        mask_words(mt, 0, w[0], w[1]);
        mask_words(mt, 1, w[2], w[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sa[4 * q + 0] = keep_if_byte<0>(w[q], sa[4 * q + 0]);
          sa[4 * q + 1] = keep_if_byte<1>(w[q], sa[4 * q + 1]);
          sa[4 * q + 2] = keep_if_byte<2>(w[q], sa[4 * q + 2]);
          sa[4 * q + 3] = keep_if_byte<3>(w[q], sa[4 * q + 3]);
        }
        return (w[0] | w[1] | w[2] | w[3]) != 0u;
      } else if constexpr (MASK == kMaskNone || MASK == kMaskBits) {
        // tail or causal tile: the keys visible by index (key < kend, and key <= qi when causal)
        // are a prefix of each run of 8 consecutive keys, so each run's visibility is the low
        // min(max(lim - first key, 0), 8) bits; then the packed mask, then the bit select
        const int lim = p.causal ? min(kend, qi + 1) : kend;
        const int rel = lim - (k0 + 32 * mt + kl);
        const int n0 = min(max(rel, 0), 8), n1 = min(max(rel - 16, 0), 8);
        uint32_t vis = ((1u << n0) - 1u) | (((1u << n1) - 1u) << 8);
        if constexpr (MASK == kMaskBits) vis &= mw >> (16 * mt);
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[r] = keep_if_bit(vis, r, sa[r]);
        return vis != 0u;
      } else {
        bool vis[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * mt + 16 * (r >> 3) + kl + (r & 7);
          vis[r] = (key < kend) & (!p.causal | (key <= qi));
        }
        if constexpr (MASK != kMaskNone) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            uint32_t lo, hi;
            mask_words(mt, hf, lo, hi);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint32_t byte = (j < 4 ? (lo >> (8 * j)) : (hi >> (8 * (j - 4)))) & 0xFFu;
              vis[8 * hf + j] = vis[8 * hf + j] & (byte != 0u);
            }
          }
        }
        bool any = false;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sa[r] = vis[r] ? sa[r] : kNegInf;
          any = any | vis[r];
        }
        return any;
      }
    };
    // Weights of one 32-key block against reference mu, packed in place as the two B operands
    // of the P.V product (no lane exchange); returns their FP32 sum (the unrounded weights).
    auto weights = [&](const f32x16& sa, float mu, u32x4 (&pb)[2]) {
      float ps = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        float pw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pw[j] = fast_exp2(fmaf(sa[8 * k2 + j], c, -mu));   // masked: 2^-inf = 0
          ps += pw[j];
        }
        pb[k2] = u32x4{E::pack2(pw[0], pw[1]), E::pack2(pw[2], pw[3]),
                       E::pack2(pw[4], pw[5]), E::pack2(pw[6], pw[7])};
      }
      return ps;
    };
    auto block_max = [&](const f32x16& sa) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[r]);
      return xor32_max(mx) * c;                        // the other 16 keys of the block
    };
    // Softmax of one block, in two parts: start() masks and computes the weights against the
    // current reference; finish() is the lazy-rescale test, which the caller places after the
    // weights.  Only when some weight of the wave could exceed 2^TAU is the reference raised to
    // the block maximum, the state rescaled and the block redone (rare, wave-uniform).  The test
    // needs no block maximum: a lane's weight sum above 2^TAU (every weight is at most the sum,
    // so a pass keeps each weight <= 2^TAU), or no reference yet while some key of the block is
    // visible (a row with nothing visible so far keeps no reference and never raises it).  Once
    // a visible key has set the reference (so l >= 1), weights that underflow to 0 are
    // negligible.
    struct BlockSm { float ps; bool any; };
    auto sm_start = [&](int mt, f32x16& sa, u32x4 (&pb)[2], auto masked_c) {
      BlockSm st;
      st.any = mask_block(mt, sa, masked_c);
      st.ps = weights(sa, (m_run == kNegInf) ? 0.f : m_run, pb);
      return st;
    };
    auto sm_finish = [&](BlockSm st, const f32x16& sa, u32x4 (&pb)[2], auto) {
      ATTN_PIN(st.ps);
      const bool raise = __builtin_amdgcn_ballot_w64((st.ps > kTauPow) | ((m_run == kNegInf) & st.any)) != 0;
      if (raise) {
        const float m_new = fmaxf(m_run, block_max(sa));
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);   // 0 from empty
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
        st.ps = weights(sa, (m_run == kNegInf) ? 0.f : m_run, pb);
      }
      l_run += st.ps;
    };

    auto tile_body = [&](auto masked_c) {
      u32x4 va[2][DT];
      u32x4 pb[2];
      if constexpr (MT >= 2) {
        // Software pipeline over the MT blocks of the tile: phase k issues the matrix work
        // S_{k+1} = K_{k+1} Q^T and O += V_{k-1} P_{k-1} and, on the vector ALUs meanwhile,
        // softmax(S_k), which depends on neither:
        //   S_0;  [S_1 || sm(S_0)];  [S_2, O += V_0 P_0 || sm(S_1)];  ...;  O += V_{MT-1} P_{MT-1}
        u32x4 kf[KSTEPS];
        u32x4 pb_prev[2];
        read_k(0, kf);
        f32x16 s_cur = qk(kf);
        // S_0 completes on its own: otherwise the scheduler interleaves S_1 with it and leaves
        // no matrix work to overlap softmax(S_0)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k <= MT; ++k) {
          f32x16 s_nxt = f32x16{};
          if (k + 1 < MT) read_k(k + 1, kf);
          if (k >= 1) read_v(k - 1, va);
          if (k + 1 < MT) s_nxt = qk(kf);
          if (k >= 1) pv(va, pb_prev);
          if (k < MT) {
            BlockSm st = sm_start(k, s_cur, pb, masked_c);
            const int n_mfma = (k + 1 < MT ? KSTEPS : 0) + (k >= 1 ? 2 * DT : 0);
            if (n_mfma > KSTEPS) {
#pragma unroll
              for (int i = 0; i < n_mfma; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
              }
            } else {
#pragma unroll
              for (int i = 0; i < n_mfma; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
              }
            }
            sm_finish(st, s_cur, pb, masked_c);
            pb_prev[0] = pb[0];
            pb_prev[1] = pb[1];
            s_cur = s_nxt;
          }
        }
      } else {                    // one block at a time (BN = 32)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          u32x4 kfa[KSTEPS];
          read_k(mt, kfa);
          f32x16 sa = qk(kfa);
          BlockSm st = sm_start(mt, sa, pb, masked_c);
          sm_finish(st, sa, pb, masked_c);
          read_v(mt, va);
          pv(va, pb);
        }
      }
    };
    // ---- V8: both 32-key blocks of the tile are turned into weights first (the FP8 product
    // consumes all 64 keys at once), so the lazy-rescale test is taken per tile, on the lane's
    // weight sum over the tile (and on no reference yet while a key is visible).  Weights <= 2^TAU = 256
    // lie inside E4M3's range (448), so the round-to-nearest-even conversion never saturates.
    auto weights8 = [&](const f32x16& sa, float mu, i32x8& pb8, int slot) {
      float ps = 0.f;
      float pw[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pw[r] = fast_exp2(fmaf(sa[r], c, -mu));
        ps += pw[r];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pw[4 * i], pw[4 * i + 1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pw[4 * i + 2], pw[4 * i + 3], w, true);
        pb8[4 * slot + i] = w;
      }
      return ps;
    };
    // block mt of the tile into slot (mt % 2) of the 64-key operand pb8
    auto sm_start8 = [&](int mt, f32x16& sa, i32x8& pb8, auto masked_c) {
      BlockSm st;
      st.any = mask_block(mt, sa, masked_c);
      st.ps = weights8(sa, (m_run == kNegInf) ? 0.f : m_run, pb8, mt & 1);
      return st;
    };
    auto read_v8 = [&](int dt, int half) {   // keys 64 half .. 64 half + 63 of the tile
      typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
      i32x8 va;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vaddr8[dt] + S * TILEV + 64 * D * half + 16 * cc * D));
        va[2 * cc] = w[0];
        va[2 * cc + 1] = w[1];
      }
      return va;
    };
    // the rescale test of one 64-key operand on both of its blocks' weight sums; a raise rescales
    // the state and redoes both blocks' weights
    auto vote8 = [&](BlockSm& a, BlockSm& b, const f32x16& sa, const f32x16& sb, i32x8& pb8) {
      ATTN_PIN(a.ps);
      ATTN_PIN(b.ps);
      const bool raise =
          __builtin_amdgcn_ballot_w64((a.ps + b.ps > kTauPow) | ((m_run == kNegInf) & (a.any | b.any))) != 0;
      if (raise) {
        const float m_new = fmaxf(m_run, fmaxf(block_max(sa), block_max(sb)));
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);   // 0 from empty
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
        const float mu = (m_run == kNegInf) ? 0.f : m_run;
        a.ps = weights8(sa, mu, pb8, 0);
        b.ps = weights8(sb, mu, pb8, 1);
      }
      l_run += a.ps + b.ps;
    };
    auto pv8 = [&](const i32x8& pb8, int half) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        // operand formats: A (V^T) E4M3 (0) or E5M2 (1), B (P) E4M3 (0)
        oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(read_v8(dt, half), pb8, oacc[dt], V8 == 2 ? 1 : 0, 0, 0, 0, 0, 0);
    };
    auto tile_body8 = [&](auto masked_c) {
      u32x4 kf[KSTEPS];
      read_k(0, kf);
      f32x16 s0 = qk(kf);
      __builtin_amdgcn_sched_barrier(0);
      read_k(1, kf);
      f32x16 s1 = qk(kf);
      i32x8 pbA;
      BlockSm st0 = sm_start8(0, s0, pbA, masked_c);
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
      }
      if constexpr (MT == 2) {
        BlockSm st1 = sm_start8(1, s1, pbA, masked_c);
        vote8(st0, st1, s0, s1, pbA);
        pv8(pbA, 0);
      } else {
        // 128-key tiles: the product of keys 0..63 runs beside block 2's softmax, so only
        // block 3's softmax has no matrix work of its own wave beside it:
        //   S_0; [S_1 || sm(S_0)]; [S_2 || sm(S_1)]; test; [O += V P_01, S_3 || sm(S_2)];
        //   sm(S_3); test; O += V P_23
        static_assert(MT == 4, "64- or 128-key tiles");
        read_k(2, kf);
        f32x16 s2 = qk(kf);
        BlockSm st1 = sm_start8(1, s1, pbA, masked_c);
#pragma unroll
        for (int i = 0; i < KSTEPS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        }
        vote8(st0, st1, s0, s1, pbA);
        pv8(pbA, 0);
        read_k(3, kf);
        f32x16 s3 = qk(kf);
        i32x8 pbB;
        BlockSm st2 = sm_start8(2, s2, pbB, masked_c);
#pragma unroll
        for (int i = 0; i < KSTEPS + DT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        BlockSm st3 = sm_start8(3, s3, pbB, masked_c);
        vote8(st2, st3, s2, s3, pbB);
        pv8(pbB, 1);
      }
    };
    if constexpr (V8) {
      if (need_tail || need_causal) tile_body8(std::true_type{});
      else tile_body8(std::false_type{});
    } else {
      if (need_tail || need_causal) tile_body(std::true_type{});
      else tile_body(std::false_type{});
    }
  };
#undef ATTN_PIN

#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < ntiles) issue_tile(i, i);
  // NSTAGE tiles per iteration, so that the LDS stage of every operand read is a constant
  for (int t = 0; t < ntiles; t += NSTAGE) {
    do_tile(t, stage_t<0>{});
    if (t + 1 < ntiles) do_tile(t + 1, stage_t<1>{});
    if constexpr (NSTAGE == 3)
      if (t + 2 < ntiles) do_tile(t + 2, stage_t<2>{});
  }

  if constexpr (BLK == 1) load_q(qb_idx, qn);   // the pair's second block

  // ---- epilogue: finish the denominator over the lane pair, normalise, store
  const float l_all = xor32_sum(l_run);
  const float inv = l_all == 0.f ? 0.f : (V8 ? p.v_scale : 1.f) / l_all;   // V8: V's scale folded in
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
  };
  if constexpr (PAIR) {
    if (2 * qb_idx != p.n_qblocks - 1) {
      run_block(qb_first, std::integral_constant<int, 1>{});
      __syncthreads();   // every wave done with the first block's stages before they are refilled
      run_block(qb_idx, std::integral_constant<int, 2>{});
    } else {   // the middle block of an odd count runs alone
      run_block(qb_first, std::integral_constant<int, 0>{});
    }
  } else {
    run_block(qb_first, std::integral_constant<int, 0>{});
  }
}


// ---- host-side dispatch -------------------------------------------------------------------
// D = 128 runs eight waves (256 query rows) per workgroup, one workgroup per CU: each K/V tile
// staged into LDS then serves twice as many queries as with four waves.  Smaller D run four
// waves, two or more workgroups per CU.
template <int D> constexpr int fwd_waves() { return D == 128 ? 8 : 4; }

// Causal launches of the eight-wave kernel pair query blocks (PAIR); the pairing instantiation
// is separate so that the others keep their single-block code.
template <typename T, int D, int BN, int MASK, bool SPLIT, int WAVES, int V8 = 0>
inline hipError_t launch_fwd_t(const FwdParams& p0, hipStream_t s) {
  constexpr int NSTAGES = WAVES == 8 && BN <= 64 ? 3 : 2;
  FwdParams p = p0;
  p.n_qblocks = (p.Nq + WAVES * kRowsPerWave - 1) / (WAVES * kRowsPerWave);
  const int64_t units = (int64_t)p.H * p.B * p.P;
  if constexpr (WAVES == 8 && !SPLIT) {
    if (p.causal && p.n_qblocks > 1) {
      dim3 grid((unsigned)(units * ((p.n_qblocks + 1) / 2)));
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, MASK, SPLIT, WAVES, NSTAGES, V8, true>), grid, dim3(64 * WAVES), 0, s, p);
      return hipGetLastError();
    }
  }
  dim3 grid((unsigned)(units * p.n_qblocks));
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, MASK, SPLIT, WAVES, NSTAGES, V8>), grid, dim3(64 * WAVES), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D, int BN>
inline hipError_t launch_fwd_mask(const FwdParams& p, bool split, hipStream_t s) {
  constexpr int W = fwd_waves<D>();
  const int mask = p.mask_bits ? kMaskBits : (p.mask == nullptr ? kMaskNone : (p.mask_lds ? kMaskLds : kMaskGlobal));
  if (split) {   // no split entry point takes a packed mask
    if (mask == kMaskLds) return launch_fwd_t<T, D, BN, kMaskLds, true, W>(p, s);
    if (mask == kMaskGlobal) return launch_fwd_t<T, D, BN, kMaskGlobal, true, W>(p, s);
    return launch_fwd_t<T, D, BN, kMaskNone, true, W>(p, s);
  }
  if (mask == kMaskBits) return launch_fwd_t<T, D, BN, kMaskBits, false, W>(p, s);
  if (mask == kMaskLds) return launch_fwd_t<T, D, BN, kMaskLds, false, W>(p, s);
  if (mask == kMaskGlobal) return launch_fwd_t<T, D, BN, kMaskGlobal, false, W>(p, s);
  return launch_fwd_t<T, D, BN, kMaskNone, false, W>(p, s);
}

}  // namespace attn
