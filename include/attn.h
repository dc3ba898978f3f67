/*
 * attn.h -- C ABI of libattn.so: streaming (online-softmax) attention for AMD MI355X (gfx950).
 *
 * Operations, each a hand-written HIP kernel enqueued on the caller's stream:
 *
 *   attn_fwd         out = softmax(Q K^T / sqrt(D)) V over visible keys, computed tile by tile
 *                    with the online-softmax recurrence (running max m, FP32 denominator l, FP32
 *                    numerator rescaled by alpha = exp(m - m')), never forming the N x N scores.
 *                    Sources: triton-cuda-lab workshop "A3. Tiled attention with online
 *                    normalization", sections "Keep three quantities for each query row" and
 *                    "Masks that preserve the recurrence"; Tylo.jl "Streaming attention and
 *                    online state", sections "Online statistics" and "Attention as a consumer".
 *   attn_fwd_splitk  the same recurrence over P contiguous key partitions, writing each
 *                    partition's locally normalised O_p / l_p and its base-2 log-sum-exp to a
 *                    workspace.  Source: Modular MAX "fa4_splitk_combine", workspace layout.
 *   attn_combine     the LSE-weighted merge of such a workspace.  Source: Modular MAX
 *                    "fa4_splitk_combine", per-row-head formulas (base 2 throughout).
 *   attn_fwd_splitk_fused   attn_fwd_splitk and attn_combine in one launch (the last
 *                    workgroup of each row-head merges).
 *   attn_fwd_splitk_noalloc  attn_fwd_splitk and attn_combine with the workspace in the
 *                    library's static device memory, for callers that cannot allocate.
 *   attn_softmax_rows        standalone row softmax (streaming, registers or three-pass)
 *                    with the all-masked conventions of Tylo.jl "Register fragments and
 *                    logical axes", section "Worked softmax".
 *   attn_fwd_fp8v    attn_fwd with V as E4M3 or E5M2 and P rounded to E4M3 for the FP8
 *                    matrix cores.
 *   attn_round       FP32 -> bf16 / fp16 / E4M3 with the conversion the kernels apply to the
 *                    probabilities and to the output (exposed so it can be checked bit by bit).
 *   attn_mask_pack   a byte mask re-encoded as one bit per (query, key), in the order the
 *                    attention kernels hold scores in their registers; attn_fwd_packed is
 *                    attn_fwd reading that encoding (one 32-bit word per lane per 64 keys
 *                    instead of 64 bytes), for masks used more than once or read by many heads.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library allocates
 *     nothing, keeps no state between calls and may be called from several threads at once
 *     (attn_fwd_splitk_noalloc excepted: it keeps its workspace in the library; see there).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous: ATTN_OK
 *     means "arguments valid, kernels enqueued".  A fault inside a kernel surfaces at the
 *     caller's next synchronisation on that stream.
 *   - On any non-OK return nothing has been enqueued and nothing written;
 *     attn_last_error() returns a message for the calling thread.  No C++ exception crosses
 *     this boundary.
 *   - Layouts are contiguous, D fastest: q and out are [B, Nq, H, D]; k and v are [B, Nkv, H, D].
 *     A row-head is one query row of one head, rh = (b * Nq + i) * H + h.
 *   - Attention entry points: q, k, v share one element type (ATTN_BF16 or ATTN_FP16); `out` uses it too,
 *     rounded to nearest even.  Scores, the softmax state, accumulation and every LSE are FP32.
 *     The weights p are rounded to the input type (nearest even) before the P.V product while
 *     the denominator sums the unrounded FP32 p (Tylo "Attention as a consumer").
 *   - The score scale is fixed at 1/sqrt(D).
 *   - Visibility of key j to query i: j < Nkv, and (causal == 0 or j <= i), and
 *     (mask == NULL or mask[i * Nkv + j] != 0).  The mask is a row-major uint8 [Nq, Nkv] array,
 *     one byte per element, shared by every batch and head.  A row with no visible key gives
 *     output 0 and LSE -inf (Tylo "Online statistics", all-masked rows).
 *   - Supported head dimensions D: 16, 32, 64, 128, 256.  B, H, N >= 1.
 *   - q, k, v, out and o_partial must be 16-byte aligned (128-bit loads and stores).
 *   - Input values must be finite; NaN or infinite inputs are outside the contract.
 */
#ifndef STREAMING_ATTN_H
#define STREAMING_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 2
#define ATTN_P_MAX 256 /* largest split count: one partition per MI355X compute unit */
#define ATTN_TICKET_STRIDE 32 /* uint32 slots per row-head in a fused-decode ticket array (128 B) */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20) /* per-GPU workspace of attn_fwd_splitk_noalloc */

enum attn_dtype {
  ATTN_BF16 = 0,
  ATTN_FP16 = 1,
  ATTN_FP32 = 2,     /* combine / softmax only */
  ATTN_FP8_E4M3 = 3, /* V of attn_fwd_fp8v; attn_round target */
  ATTN_FP8_E5M2 = 4  /* V of attn_fwd_fp8v */
};

enum attn_status {
  ATTN_OK = 0,
  ATTN_E_NULL = 1,        /* a required pointer is NULL */
  ATTN_E_SHAPE = 2,       /* a size is < 1, sizes overflow, or causal with Nq != Nkv */
  ATTN_E_UNSUPPORTED = 3, /* D, dtype, P or block size outside the supported set */
  ATTN_E_ALIGN = 4,       /* a pointer lacks the required alignment */
  ATTN_E_WORKSPACE = 5,   /* split-K workspace pointers missing */
  ATTN_E_HIP = 6          /* the HIP runtime refused a launch; see attn_last_error() */
};

/*
 * attn_fwd -- square attention (Nq = Nkv = N).
 *   q, k, v   [B, N, H, D] of `dtype`, read only.
 *   out       [B, N, H, D] of `dtype`, written: O_i = sum_j p_ij v_j / l_i, 0 for an all-masked row.
 *   lse       nullable; [B, N, H] float32, written: NATURAL-log log-sum-exp of the scaled
 *             logits over the visible keys, -inf for an all-masked row.
 *   causal    0 or 1 (key j visible to query i only if j <= i; the diagonal is included).
 *   mask      nullable; uint8 [N, N] as above.
 *   dtype     ATTN_BF16 or ATTN_FP16.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N,
             int D, int causal, const uint8_t* mask, int dtype, void* stream);

/*
 * attn_fwd_splitk -- the recurrence over P key partitions (Modular MAX "fa4_splitk_combine").
 *   Partition p covers keys [p*c, min((p+1)*c, Nkv)) with c = ceil(Nkv / P); a partition may be
 *   empty, or have no key visible to a row.
 *   q            [B, Nq, H, D]; k, v [B, Nkv, H, D] of `dtype`.
 *   o_partial    [P, B*Nq, H, D] float32, written: the partition's locally normalised O_p / l_p,
 *                exactly 0 when the partition has no visible key for that row-head.
 *   lse_partial  [P, B*Nq, H] float32, written: BASE-2 log-sum-exp m2 + log2(l_p), where m2 is
 *                the running maximum of the logits in log2 units (logit * log2(e)); -inf when
 *                the partition has no visible key for that row-head.
 *   out, lse     nullable.  When out != NULL, attn_combine(o_partial, lse_partial, out, lse, P,
 *                B*Nq, H, D, dtype, stream) is enqueued right after, in stream order.
 *   causal       requires Nq == Nkv (rectangular causal has no defined offset: ATTN_E_SHAPE).
 *   P            1 .. ATTN_P_MAX.
 *   Nq == 1 runs a bandwidth-bound decode kernel (one workgroup per row-head and partition);
 *   Nq > 1 runs the tiled matrix-core kernel once per partition.
 */
int attn_fwd_splitk(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                    int Nq, int Nkv, int D, int causal, const uint8_t* mask, int P, float* o_partial,
                    float* lse_partial, int dtype, void* stream);

/*
 * attn_fwd_splitk_noalloc -- attn_fwd_splitk with out != NULL (the split-K producer, then the
 *   combine, on the same kernels), for callers that cannot allocate device memory: code under
 *   HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The call allocates
 *   and frees nothing (no hipMalloc, hipFree or allocating library routine): the workspace
 *   (o_partial [P, B*Nq, H, D] float32, then lse_partial [P, B*Nq, H] float32 at the next
 *   256-byte boundary) lives in a static device array of ATTN_NOALLOC_SCRATCH_BYTES inside the
 *   library, one per GPU, held until the process ends; its address is looked up on the first call
 *   on each device.
 *   Arguments: as attn_fwd_splitk without o_partial and lse_partial; out is REQUIRED.
 *   Limit: P * B * Nq * H * D * 4, rounded up to 256, plus P * B * Nq * H * 4 must not exceed
 *   ATTN_NOALLOC_SCRATCH_BYTES (64 MiB: the decode shape B8 H32 D128 fits up to P = 256),
 *   else ATTN_E_WORKSPACE and nothing is enqueued.
 *   Sharing: every call on one GPU uses that GPU's array, which keeps the last call's contents.
 *   Each call writes every workspace entry before its combine reads it, so nothing needs
 *   clearing, but calls that overlap in time on one GPU (other streams, other host threads)
 *   race on the array: the caller must order them.  `stream` must belong to the current device
 *   (ATTN_E_HIP otherwise).
 *   Errors: those of attn_fwd_splitk and attn_combine, plus ATTN_E_WORKSPACE for the limit.
 */
int attn_fwd_splitk_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                            int Nq, int Nkv, int D, int causal, const uint8_t* mask, int P, int dtype,
                            void* stream);

/*
 * attn_fwd_splitk_fused -- attn_fwd_splitk followed by the combine, in ONE launch (the CDNA4
 *   counterpart of Modular MAX "fa4_splitk_combine"'s overlap of the combine with the producer's
 *   tail).  Each (row-head, partition) workgroup writes its workspace entry as attn_fwd_splitk
 *   does, makes it visible device-wide and increments its row-head's ticket; the workgroup that
 *   takes the last ticket merges the P entries with attn_combine's formulas, writes out / lse and
 *   resets the ticket to 0.  Every row-head runs on the bandwidth-bound decode kernel, so this is
 *   meant for few-query (decode) shapes.
 *   Arguments as attn_fwd_splitk, except:
 *   out          REQUIRED, [B, Nq, H, D] of `dtype`.
 *   lse          nullable; [B, Nq, H] float32, natural log.
 *   tickets      REQUIRED, uint32 [B * Nq * H * ATTN_TICKET_STRIDE], 4-byte aligned,
 *                caller-owned.  Row-head rh counts in tickets[rh * ATTN_TICKET_STRIDE]; the other
 *                slots are padding that keeps every counter on its own 128-byte line (counters
 *                that share a line serialise their atomics in the memory system).  It must hold 0
 *                in every counter before the first call (e.g. one hipMemset at allocation); a call
 *                that runs to completion leaves it at 0 again, so it is reusable without clearing.
 *                Two calls that overlap in time (different streams) must not share it.
 *   Errors: ATTN_E_WORKSPACE if o_partial, lse_partial or tickets is NULL; otherwise as
 *   attn_fwd_splitk and attn_combine.
 */
int attn_fwd_splitk_fused(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                          int H, int Nq, int Nkv, int D, int causal, const uint8_t* mask, int P,
                          float* o_partial, float* lse_partial, uint32_t* tickets, int dtype,
                          void* stream);

/*
 * attn_combine -- merge a split-K workspace (Modular MAX "fa4_splitk_combine"):
 *   for each row-head rh of rows*heads:  m* = max_p lse_p;  G = log2(sum_p 2^(lse_p - m*)) + m*;
 *   scale_p = 2^(lse_p - G);  out[rh, d] = sum_p scale_p * o_partial[p, rh, d].
 *   o_partial    [P, rows, heads, depth] float32 (locally normalised partials), read only.
 *   lse_partial  [P, rows, heads] float32, base 2, read only.  -inf marks an empty partition,
 *                which contributes nothing; if every partition is -inf, out = 0 and lse = -inf.
 *   out          [rows, heads, depth] of out_dtype (ATTN_BF16, ATTN_FP16 or ATTN_FP32).
 *   lse_out      nullable; [rows, heads] float32, NATURAL log (G * ln 2), comparable with the
 *                lse of attn_fwd.
 *   depth        16, 32, 64, 128 or 256.  P in 1 .. ATTN_P_MAX.  P = 4, 8 and 16 run fully
 *                unrolled instantiations; any other P runs the runtime-P instantiation.
 */
int attn_combine(const float* o_partial, const float* lse_partial, void* out, float* lse_out, int P,
                 int rows, int heads, int depth, int out_dtype, void* stream);

/*
 * attn_softmax_rows -- standalone row softmax, y[r, j] = exp(x[r, j] - m_r) / sum_j' exp(x[r, j'] - m_r)
 *   with m_r the row maximum, under the all-masked conventions of Tylo.jl "Register fragments and
 *   logical axes", section "Worked softmax": x = -inf marks a masked entry (y = 0 there), and a row
 *   whose entries are all -inf gives y = 0 throughout (never NaN).  Other values must be finite.
 *   x, y      row-major [rows, n] of `dtype` (ATTN_BF16, ATTN_FP16 or ATTN_FP32), aligned to the
 *             element size; y is rounded to nearest even for 16-bit types.  x == y (in place) is
 *             allowed; other overlap is not.
 *   method    ATTN_SOFTMAX_STREAMING: two passes with four values per lane per step, whatever n
 *               (statistics streamed first, logits reread to write; Tylo "Streaming attention and
 *               online state", section "Online statistics");
 *             ATTN_SOFTMAX_REGISTERS: the whole row held in registers, one read: one wave per
 *               row for n <= 4096, a 16-wave workgroup per row for 4096 < n <= 65536;
 *             ATTN_SOFTMAX_THREE_PASS: a scalar loop over max, sum of exponentials, write.
 *             All three compute the same function; they differ in memory traffic and registers.
 *   Errors: ATTN_E_NULL, ATTN_E_SHAPE (rows or n < 1, sizes overflow), ATTN_E_UNSUPPORTED (dtype,
 *   method, or n > 65536 with the registers method), ATTN_E_ALIGN.
 */
enum attn_softmax_method { ATTN_SOFTMAX_STREAMING = 0, ATTN_SOFTMAX_REGISTERS = 1, ATTN_SOFTMAX_THREE_PASS = 2 };
int attn_softmax_rows(const void* x, void* y, int64_t rows, int n, int dtype, int method, void* stream);

/*
 * attn_round -- y[i] = x[i] rounded to bf16, fp16 or E4M3, to nearest with ties to even, by the
 *   packed conversion the attention kernels use for the probabilities before the second product
 *   and for the stored output.
 *   bf16 / fp16 (Tylo.jl "Streaming attention and online state", section "Same-lane conversion":
 *   signed zeros and infinities kept, NaN stays NaN, no saturation and no flush to zero; Tylo.jl
 *   "Register fragments and logical axes", section "Logical types and register packing": the
 *   packed word): values beyond the largest finite value become +-inf.
 *   ATTN_FP8_E4M3 (the same section's 8-bit rule): saturation to +-448 instead, infinities give
 *   +-448, subnormals kept, NaN gives a NaN code.
 *   x      n FP32 values (device, 4-byte aligned);  y  n results of dtype's size (device, aligned
 *          to it).
 *   dtype  ATTN_BF16, ATTN_FP16 or ATTN_FP8_E4M3.  n = 0 enqueues nothing.
 *   Errors: ATTN_E_SHAPE (n < 0), ATTN_E_NULL, ATTN_E_UNSUPPORTED (dtype), ATTN_E_ALIGN.
 */
int attn_round(const float* x, void* y, int64_t n, int dtype, void* stream);

/* Extended forward call for tests and tuning: every attn_fwd argument plus the key-tile width
 * and the packed mask of attn_fwd_packed (at most one of mask and mask_bits). */
struct attn_fwd_args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;          /* nullable */
  const uint8_t* mask; /* nullable */
  int B, H, N, D;
  int causal;
  int dtype;
  int block_n;         /* key-tile width: 0 = library default, else 32 or 64 (32 only for D <= 64) */
  const uint32_t* mask_bits; /* nullable; as attn_fwd_packed, packed with the same causal flag */
};
int attn_fwd_ex(const struct attn_fwd_args* a, void* stream);

/*
 * attn_fwd_fp8v -- attn_fwd with V in 8-bit floating point and the second product (P.V) on the
 *   FP8 matrix cores.  Element types from Tylo.jl "Register fragments and logical axes", section
 *   "Logical types and register packing" (Float8E4M3 and Float8E5M2: four 8-bit values per
 *   32-bit register; FP32 conversion to nearest even, saturating to the largest finite value);
 *   the recurrence is attn_fwd's.  The value of V[b, j, h, d] is decode(v[b, j, h, d]) * v_scale
 *   in the format v_format names.  Each
 *   probability is rounded from FP32 to E4M3 (nearest even; it is at most 256, inside E4M3's
 *   range) before the product, while the denominator l keeps the unrounded FP32 weights (the
 *   rounding-before-PV rule of Tylo.jl "Streaming attention and online state", section
 *   "Attention as a consumer").  Q K^T stays in q/k's type.
 *   q, k, out  [B, N, H, D] bf16 or fp16 (dtype), 16-byte aligned; D must be 128.
 *   v          [B, N, H, D] 8-bit codes, one byte per element, 16-byte aligned; codes must be
 *              finite.
 *   v_format   ATTN_FP8_E4M3 (S.EEEE.MMM, bias 7, no infinities, S.1111.111 = NaN) or
 *              ATTN_FP8_E5M2 (S.EEEEE.MM, bias 15, IEEE-like).
 *   v_scale    finite FP32 scale of V (1.0 when V is stored unscaled).
 *   lse, causal, mask, stream: as attn_fwd (lse is the LSE of the scores, unaffected by v_scale).
 *   Errors: those of attn_fwd; ATTN_E_UNSUPPORTED also for D != 128, another v_format or a
 *   non-finite v_scale.
 */
int attn_fwd_fp8v(const void* q, const void* k, const uint8_t* v, int v_format, float v_scale, void* out,
                  float* lse, int B, int H, int N, int D, int causal, const uint8_t* mask, int dtype, void* stream);

/*
 * Packed masks.  The mask semantics are attn_fwd's (a key is visible where the byte is nonzero:
 * triton-cuda-lab workshop "A3. Tiled attention with online normalization", section "Masks that
 * preserve the recurrence"); the encoding is this library's, chosen so that each lane of a
 * 64-wide wavefront loads the visibility of exactly the scores it holds.  With Nq x Nkv bytes
 * of mask, ATTN_MASK_BITS_WORDS(Nq, Nkv) uint32 words: for row group g (rows 32 g .. 32 g + 31),
 * key group c (keys 64 c .. 64 c + 63) and lane l (0 .. 63), word (g * ceil(Nkv / 64) + c) * 64
 * + l has bit b (0 .. 31) set iff row 32 g + l % 32 and key
 *     64 c + 32 (b / 16) + 16 ((b % 16) / 8) + 8 (l / 32) + b % 8
 * are inside the mask and its byte is nonzero.
 */
#define ATTN_MASK_BITS_WORDS(Nq, Nkv) \
  ((((int64_t)(Nq) + 31) / 32) * (((int64_t)(Nkv) + 63) / 64) * 64)

/*
 * attn_mask_pack -- encode a byte mask as above.
 *   mask    uint8 [Nq, Nkv] row-major, device, read only (any alignment).
 *   Nq, Nkv >= 1.
 *   causal  0: every word is written.  1 (requires Nq == Nkv): only the groups a causal forward
 *           reads are written, those with 64 c <= 32 g + 31; the mask bytes above them are not
 *           read and the other words are left as they were.  Bits packed with causal = 1 serve
 *           causal forward calls only.
 *   bits    ATTN_MASK_BITS_WORDS(Nq, Nkv) uint32, device, 4-byte aligned, written.
 *   Errors: ATTN_E_NULL, ATTN_E_SHAPE (sizes, causal with Nq != Nkv), ATTN_E_ALIGN (bits),
 *   ATTN_E_HIP.
 */
int attn_mask_pack(const uint8_t* mask, int Nq, int Nkv, int causal, uint32_t* bits, void* stream);

/*
 * attn_fwd_packed -- attn_fwd with the mask given as attn_mask_pack's bits (of the N x N mask,
 *   packed with the same causal flag); mask_bits is required.  Results are bit for bit those of
 *   attn_fwd with the byte mask.  Other arguments and errors: as attn_fwd; ATTN_E_NULL without
 *   mask_bits, ATTN_E_ALIGN unless it is 4-byte aligned.
 */
int attn_fwd_packed(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N,
                    int D, int causal, const uint32_t* mask_bits, int dtype, void* stream);

/* Message describing the calling thread's last non-OK return ("" if none). */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STREAMING_ATTN_H */
