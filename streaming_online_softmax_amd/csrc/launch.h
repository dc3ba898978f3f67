// launch.h -- kernel parameter blocks and launchers (internal to libattn.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int ATTN_P_MAX_DEV = 256;   // largest split count (one partition per compute unit)
constexpr int ATTN_TICKET_STRIDE_DEV = 32;   // uint32 slots per row-head ticket: one 128-byte line each

// Tiled matrix-core forward (attn_fwd, and the split-K producer when Nq > 1).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;            // [B, Nq, H, D] input dtype (unsplit)
  float* lse;           // [B, Nq, H] natural log, nullable (unsplit)
  float* o_partial;     // [P, B*Nq, H, D] (split)
  float* lse_partial;   // [P, B*Nq, H] base 2 (split)
  const uint8_t* mask;  // [Nq, Nkv] or null
  int B, H, Nq, Nkv;
  int causal;
  int P;                // 1 when unsplit
  int chunk;            // keys per partition (split)
  int n_qblocks;        // ceil(Nq / query rows per workgroup); set by the launcher
  int mask_vec;         // mask rows may be read 8 bytes at a time
  int mask_lds;         // mask tiles may be staged into LDS 16 bytes at a time (row starts
                        // 16-byte aligned, (Nq + 256) * Nkv < 2^32)
  float scale_log2;     // log2(e) / sqrt(D)
  float v_scale;        // 8-bit V (attn_fwd_fp8v): value = decoded code * v_scale
  const uint32_t* mask_bits;   // packed mask (unsplit only; replaces mask): [ceil(Nq/32)][n_kgroups][64]
  int n_kgroups;        // ceil(Nkv / 64)
};

// Bandwidth-bound split-K decode producer (one workgroup per row-head and partition).
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  float* o_partial;
  float* lse_partial;
  const uint8_t* mask;
  int B, H, Nq, Nkv;
  int causal;
  int P;
  int chunk;
  float scale_log2;
  // fused combine (attn_fwd_splitk_fused): the last workgroup of each row-head merges the
  // workspace into out / lse; tickets[rh * ATTN_TICKET_STRIDE_DEV] counts finished partitions
  // and is returned to 0
  void* out;            // [B, Nq, H, D] input dtype
  float* lse;           // [B, Nq, H] natural log, nullable
  uint32_t* tickets;    // [B * Nq * H * ATTN_TICKET_STRIDE_DEV], counters zero on entry and exit
};

// LSE-weighted combine of a split-K workspace.
struct CombineParams {
  const float* o_partial;
  const float* lse_partial;
  void* out;
  float* lse_out;       // natural log, nullable
  int P;
  int RH;               // rows * heads
  int depth;            // elements per row-head (set by launch_combine)
};

// Standalone row softmax (attn_softmax_rows).
enum { SM_STREAM = 0, SM_REGS = 1, SM_THREE = 2 };
struct SoftmaxParams {
  const void* x;        // [rows, n] logits
  void* y;              // [rows, n] probabilities, same element type
  int64_t rows;
  int n;
};

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int BN, bool split, hipStream_t s);
// D = 256 instantiations (attn_fwd_d256.hip), called by launch_fwd
hipError_t launch_fwd_d256(const FwdParams& p, int dtype, bool split, hipStream_t s);
// D = 128, 8-bit V (v_format 0 = E4M3, 1 = E5M2), FP8 second product (p.P = 1)
hipError_t launch_fwd_fp8v(const FwdParams& p, int dtype, int v_format, hipStream_t s);
hipError_t launch_softmax_rows(const SoftmaxParams& p, int dtype, int method, bool vec, hipStream_t s);
int softmax_regs_max_n();
// FP32 -> bf16 (dtype 0), fp16 (dtype 1) or E4M3 (dtype 3, saturating), n values, with the
// kernels' packed conversions.
hipError_t launch_round(const float* x, void* y, int64_t n, int dtype, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int dtype, int D, bool fused, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, int depth, int out_dtype, hipStream_t s);
int fwd_block_m();
// attn_mask_pack: byte mask [Nq, Nkv] -> lane-order bits (include/attn.h); causal skips the
// groups above the diagonal.
hipError_t launch_mask_pack(const uint8_t* mask, int Nq, int Nkv, int causal, uint32_t* bits, hipStream_t s);

}  // namespace attn
