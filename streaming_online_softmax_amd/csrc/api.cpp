// api.cpp -- the C ABI of libattn.so: argument validation, kernel selection, launch on the
// caller's stream.  Validation happens before any HIP call, so a rejected call enqueues
// nothing, writes nothing and touches no device (the pages' rule that unsupported layouts are
// rejected rather than silently computed differently: Tylo.jl "Streaming attention and online
// state", section "Same-lane conversion"; workshop "Masks that preserve the recurrence",
// rectangular causal rejected).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "../../include/attn.h"
#include "launch.h"

static_assert(ATTN_P_MAX == attn::ATTN_P_MAX_DEV, "split bound differs between header and kernels");
static_assert(ATTN_TICKET_STRIDE == attn::ATTN_TICKET_STRIDE_DEV, "ticket stride differs between header and kernels");

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool supported_d(int D) { return D == 16 || D == 32 || D == 64 || D == 128 || D == 256; }

float scale_log2(int D) { return (float)(1.4426950408889634 / std::sqrt((double)D)); }

// Shared checks of q/k/v/out sizes.  Returns ATTN_OK or an error code (message set).
int check_qkv(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nkv, int D,
              int causal, int dtype) {
  if (!q || !k || !v) return fail(ATTN_E_NULL, "q, k and v must be non-NULL device pointers");
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return fail(ATTN_E_SHAPE, "B, H, Nq, Nkv must be >= 1 (got %d, %d, %d, %d)", B, H, Nq, Nkv);
  if (!supported_d(D)) return fail(ATTN_E_UNSUPPORTED, "head dimension D=%d not supported (16, 32, 64, 128, 256)", D);
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return fail(ATTN_E_UNSUPPORTED, "dtype %d not supported for q/k/v (ATTN_BF16 or ATTN_FP16)", dtype);
  if (causal != 0 && causal != 1) return fail(ATTN_E_SHAPE, "causal must be 0 or 1 (got %d)", causal);
  if (causal && Nq != Nkv) return fail(ATTN_E_SHAPE, "causal attention requires Nq == Nkv (got %d, %d): a rectangular causal offset is not defined", Nq, Nkv);
  const double elems_q = (double)B * Nq * H * D, elems_kv = (double)B * Nkv * H * D;
  if (elems_q > 9.0e15 || elems_kv > 9.0e15) return fail(ATTN_E_SHAPE, "tensor sizes overflow");
  if ((double)Nq * Nkv > 9.0e18) return fail(ATTN_E_SHAPE, "mask size overflows");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return fail(ATTN_E_ALIGN, "q, k and v must be 16-byte aligned");
  return ATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- the workspace of attn_fwd_splitk_noalloc: one static device array, which every GPU the
//      library runs on holds (with the code object) until the process ends.  In host code the
//      name `scratch` is only a handle for the runtime; the device address comes from
//      hipGetSymbolAddress, looked up once per device with that device current and kept here.
constexpr uint64_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device `stream` runs on, which must be the current device.
int scratch_for_stream(hipStream_t stream, uint8_t** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_E_HIP, "device ordinal %d out of range", dev);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev) return fail(ATTN_E_HIP, "the stream belongs to device %d but device %d is current", (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(ATTN_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

int do_combine(const float* o_partial, const float* lse_partial, void* out, float* lse_out, int P,
               int rows, int heads, int depth, int out_dtype, hipStream_t s) {
  attn::CombineParams cp;
  cp.o_partial = o_partial;
  cp.lse_partial = lse_partial;
  cp.out = out;
  cp.lse_out = lse_out;
  cp.P = P;
  cp.RH = rows * heads;
  return hip_status(attn::launch_combine(cp, depth, out_dtype, s), "attn_combine launch");
}

int check_combine(const float* o_partial, const float* lse_partial, void* out, float* lse_out, int P,
                  int rows, int heads, int depth, int out_dtype) {
  if (!o_partial || !lse_partial || !out) return fail(ATTN_E_NULL, "o_partial, lse_partial and out must be non-NULL");
  if (P < 1) return fail(ATTN_E_SHAPE, "P must be >= 1 (got %d)", P);
  if (P > ATTN_P_MAX) return fail(ATTN_E_UNSUPPORTED, "P=%d exceeds ATTN_P_MAX=%d", P, ATTN_P_MAX);
  if (rows < 1 || heads < 1) return fail(ATTN_E_SHAPE, "rows and heads must be >= 1");
  if ((int64_t)rows * heads > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "rows*heads exceeds 2^31-1");
  if (!supported_d(depth)) return fail(ATTN_E_UNSUPPORTED, "depth=%d not supported (16, 32, 64, 128, 256)", depth);
  if (out_dtype != ATTN_BF16 && out_dtype != ATTN_FP16 && out_dtype != ATTN_FP32) return fail(ATTN_E_UNSUPPORTED, "out_dtype %d not supported", out_dtype);
  if (!aligned(o_partial, 16)) return fail(ATTN_E_ALIGN, "o_partial must be 16-byte aligned");
  if (!aligned(lse_partial, 4) || (lse_out && !aligned(lse_out, 4))) return fail(ATTN_E_ALIGN, "LSE arrays must be 4-byte aligned");
  if (!aligned(out, 16)) return fail(ATTN_E_ALIGN, "out must be 16-byte aligned");
  return ATTN_OK;
}

int fwd_impl(const attn_fwd_args* a, hipStream_t s) {
  int rc = check_qkv(a->q, a->k, a->v, a->B, a->H, a->N, a->N, a->D, a->causal, a->dtype);
  if (rc) return rc;
  if (!a->out) return fail(ATTN_E_NULL, "out must be a non-NULL device pointer");
  if (!aligned(a->out, 16)) return fail(ATTN_E_ALIGN, "out must be 16-byte aligned");
  if (a->lse && !aligned(a->lse, 4)) return fail(ATTN_E_ALIGN, "lse must be 4-byte aligned");
  if (a->mask && a->mask_bits) return fail(ATTN_E_SHAPE, "give the mask as bytes or as packed bits, not both");
  if (a->mask_bits && !aligned(a->mask_bits, 4)) return fail(ATTN_E_ALIGN, "mask_bits must be 4-byte aligned");
  int BN = a->block_n;
  if (BN == 0) BN = 64;
  if (BN != 32 && BN != 64) return fail(ATTN_E_UNSUPPORTED, "block_n=%d not supported (32 or 64)", a->block_n);
  if (BN == 32 && a->D > 64) return fail(ATTN_E_UNSUPPORTED, "block_n=32 is built for D <= 64 only");
  const int64_t nqb = ((int64_t)a->N + attn::fwd_block_m() - 1) / attn::fwd_block_m();
  if (nqb * a->H * a->B > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "grid too large");

  attn::FwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.out = a->out; p.lse = a->lse;
  p.mask = a->mask;
  p.B = a->B; p.H = a->H; p.Nq = a->N; p.Nkv = a->N;
  p.causal = a->causal;
  p.P = 1; p.chunk = a->N;
  p.n_qblocks = (int)nqb;
  p.mask_vec = a->mask && aligned(a->mask, 8) && (a->N % 8 == 0);
  p.mask_lds = a->mask && aligned(a->mask, 16) && (a->N % 16 == 0) && ((int64_t)a->N + 256) * a->N < (1LL << 32);
  p.mask_bits = a->mask_bits;
  p.n_kgroups = (a->N + 63) / 64;
  p.scale_log2 = scale_log2(a->D);
  return hip_status(attn::launch_fwd(p, a->dtype, a->D, BN, false, s), "attn_fwd launch");
}

int splitk_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nq,
                int Nkv, int D, int causal, const uint8_t* mask, int P, float* o_partial, float* lse_partial,
                int dtype, hipStream_t s) {
  int rc = check_qkv(q, k, v, B, H, Nq, Nkv, D, causal, dtype);
  if (rc) return rc;
  if (P < 1) return fail(ATTN_E_SHAPE, "P must be >= 1 (got %d)", P);
  if (P > ATTN_P_MAX) return fail(ATTN_E_UNSUPPORTED, "P=%d exceeds ATTN_P_MAX=%d", P, ATTN_P_MAX);
  if (!o_partial || !lse_partial) return fail(ATTN_E_WORKSPACE, "o_partial and lse_partial are required");
  if (!aligned(o_partial, 16)) return fail(ATTN_E_ALIGN, "o_partial must be 16-byte aligned");
  if (!aligned(lse_partial, 4)) return fail(ATTN_E_ALIGN, "lse_partial must be 4-byte aligned");
  const int64_t RH = (int64_t)B * Nq * H;
  if (RH > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "B*Nq*H exceeds 2^31-1");
  if (out) {
    rc = check_combine(o_partial, lse_partial, out, lse, P, B * Nq, H, D, dtype);
    if (rc) return rc;
  }
  const int chunk = (int)(((int64_t)Nkv + P - 1) / P);
  const float c = scale_log2(D);
  if (Nq == 1) {
    if (RH * P > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "grid too large");
    attn::DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.o_partial = o_partial; p.lse_partial = lse_partial; p.mask = mask;
    p.B = B; p.H = H; p.Nq = Nq; p.Nkv = Nkv; p.causal = causal; p.P = P; p.chunk = chunk; p.scale_log2 = c;
    rc = hip_status(attn::launch_decode(p, dtype, D, false, s), "attn_fwd_splitk decode launch");
  } else {
    const int64_t nqb = ((int64_t)Nq + attn::fwd_block_m() - 1) / attn::fwd_block_m();
    if (nqb * H * B * P > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "grid too large");
    attn::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o_partial = o_partial; p.lse_partial = lse_partial; p.mask = mask;
    p.B = B; p.H = H; p.Nq = Nq; p.Nkv = Nkv; p.causal = causal; p.P = P; p.chunk = chunk;
    p.n_qblocks = (int)nqb;
    p.mask_vec = mask && aligned(mask, 8) && (Nkv % 8 == 0) && (chunk % 8 == 0);
    p.mask_lds = mask && aligned(mask, 16) && (Nkv % 16 == 0) && (chunk % 16 == 0) && ((int64_t)Nq + 256) * Nkv < (1LL << 32);
    p.scale_log2 = c;
    rc = hip_status(attn::launch_fwd(p, dtype, D, 64, true, s), "attn_fwd_splitk launch");
  }
  if (rc || !out) return rc;
  return do_combine(o_partial, lse_partial, out, lse, P, B * Nq, H, D, dtype, s);
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_err; }

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N,
             int D, int causal, const uint8_t* mask, int dtype, void* stream) {
  attn_fwd_args a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.mask = mask;
  a.B = B; a.H = H; a.N = N; a.D = D; a.causal = causal; a.dtype = dtype; a.block_n = 0;
  return fwd_impl(&a, (hipStream_t)stream);
}

int attn_fwd_packed(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N,
                    int D, int causal, const uint32_t* mask_bits, int dtype, void* stream) {
  if (!mask_bits) return fail(ATTN_E_NULL, "mask_bits must be a non-NULL device pointer");
  attn_fwd_args a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.mask_bits = mask_bits;
  a.B = B; a.H = H; a.N = N; a.D = D; a.causal = causal; a.dtype = dtype; a.block_n = 0;
  return fwd_impl(&a, (hipStream_t)stream);
}

int attn_mask_pack(const uint8_t* mask, int Nq, int Nkv, int causal, uint32_t* bits, void* stream) {
  if (!mask || !bits) return fail(ATTN_E_NULL, "mask and bits must be non-NULL device pointers");
  if (Nq < 1 || Nkv < 1) return fail(ATTN_E_SHAPE, "Nq and Nkv must be >= 1 (got %d, %d)", Nq, Nkv);
  if (causal != 0 && causal != 1) return fail(ATTN_E_SHAPE, "causal must be 0 or 1 (got %d)", causal);
  if (causal && Nq != Nkv) return fail(ATTN_E_SHAPE, "causal packing requires Nq == Nkv (got %d, %d)", Nq, Nkv);
  if (!aligned(bits, 4)) return fail(ATTN_E_ALIGN, "bits must be 4-byte aligned");
  if ((double)Nq * Nkv > 9.0e18) return fail(ATTN_E_SHAPE, "mask size overflows");
  if ((((int64_t)Nq + 31) / 32) * ((((int64_t)Nkv + 63) / 64 + 3) / 4) > 0x7fffffffLL)
    return fail(ATTN_E_SHAPE, "grid too large");
  return hip_status(attn::launch_mask_pack(mask, Nq, Nkv, causal, bits, (hipStream_t)stream), "attn_mask_pack launch");
}

int attn_fwd_ex(const struct attn_fwd_args* a, void* stream) {
  if (!a) return fail(ATTN_E_NULL, "args must be non-NULL");
  return fwd_impl(a, (hipStream_t)stream);
}

int attn_fwd_fp8v(const void* q, const void* k, const uint8_t* v, int v_format, float v_scale, void* out,
                  float* lse, int B, int H, int N, int D, int causal, const uint8_t* mask, int dtype, void* stream) {
  int rc = check_qkv(q, k, v, B, H, N, N, D, causal, dtype);
  if (rc) return rc;
  if (D != 128) return fail(ATTN_E_UNSUPPORTED, "attn_fwd_fp8v is built for D = 128 (got %d)", D);
  if (v_format != ATTN_FP8_E4M3 && v_format != ATTN_FP8_E5M2)
    return fail(ATTN_E_UNSUPPORTED, "v_format %d not supported (ATTN_FP8_E4M3 or ATTN_FP8_E5M2)", v_format);
  if (!std::isfinite(v_scale)) return fail(ATTN_E_UNSUPPORTED, "v_scale must be finite");
  if (!out) return fail(ATTN_E_NULL, "out must be a non-NULL device pointer");
  if (!aligned(out, 16)) return fail(ATTN_E_ALIGN, "out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(ATTN_E_ALIGN, "lse must be 4-byte aligned");
  const int64_t nqb = ((int64_t)N + 255) / 256;
  if (nqb * H * B > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "grid too large");
  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v;
  p.out = out; p.lse = lse;
  p.mask = mask;
  p.B = B; p.H = H; p.Nq = N; p.Nkv = N;
  p.causal = causal;
  p.P = 1; p.chunk = N;
  p.mask_vec = mask && aligned(mask, 8) && (N % 8 == 0);
  p.mask_lds = mask && aligned(mask, 16) && (N % 16 == 0) && ((int64_t)N + 256) * N < (1LL << 32);
  p.scale_log2 = scale_log2(D);
  p.v_scale = v_scale;
  return hip_status(attn::launch_fwd_fp8v(p, dtype, v_format == ATTN_FP8_E5M2 ? 1 : 0, (hipStream_t)stream),
                    "attn_fwd_fp8v launch");
}

int attn_fwd_splitk(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                    int Nq, int Nkv, int D, int causal, const uint8_t* mask, int P, float* o_partial,
                    float* lse_partial, int dtype, void* stream) {
  return splitk_impl(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, mask, P, o_partial, lse_partial, dtype,
                     (hipStream_t)stream);
}

int attn_fwd_splitk_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                            int Nq, int Nkv, int D, int causal, const uint8_t* mask, int P, int dtype,
                            void* stream) {
  // every argument is checked before the device is touched
  int rc = check_qkv(q, k, v, B, H, Nq, Nkv, D, causal, dtype);
  if (rc) return rc;
  if (P < 1) return fail(ATTN_E_SHAPE, "P must be >= 1 (got %d)", P);
  if (P > ATTN_P_MAX) return fail(ATTN_E_UNSUPPORTED, "P=%d exceeds ATTN_P_MAX=%d", P, ATTN_P_MAX);
  if (!out) return fail(ATTN_E_NULL, "out is required");
  if (!aligned(out, 16)) return fail(ATTN_E_ALIGN, "out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(ATTN_E_ALIGN, "lse must be 4-byte aligned");
  if ((int64_t)B * Nq * H > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "B*Nq*H exceeds 2^31-1");
  const uint64_t rh_all = (uint64_t)P * B * Nq * H;
  const uint64_t o_bytes = (rh_all * D * 4 + 255) / 256 * 256;
  const uint64_t need = o_bytes + rh_all * 4;
  if ((double)P * B * Nq * H * (D + 1) * 4.0 > 1.0e15 || need > kScratchBytes)
    return fail(ATTN_E_WORKSPACE, "workspace of %llu bytes (P*B*Nq*H*(D+1)*4, lse at a 256-byte boundary) exceeds the "
                "%llu-byte static scratch of attn_fwd_splitk_noalloc", (unsigned long long)need,
                (unsigned long long)kScratchBytes);
  uint8_t* ws = nullptr;
  rc = scratch_for_stream((hipStream_t)stream, &ws);
  if (rc) return rc;
  return splitk_impl(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, mask, P, reinterpret_cast<float*>(ws),
                     reinterpret_cast<float*>(ws + o_bytes), dtype, (hipStream_t)stream);
}

int attn_fwd_splitk_fused(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                          int H, int Nq, int Nkv, int D, int causal, const uint8_t* mask, int P,
                          float* o_partial, float* lse_partial, uint32_t* tickets, int dtype,
                          void* stream) {
  int rc = check_qkv(q, k, v, B, H, Nq, Nkv, D, causal, dtype);
  if (rc) return rc;
  if (P < 1) return fail(ATTN_E_SHAPE, "P must be >= 1 (got %d)", P);
  if (P > ATTN_P_MAX) return fail(ATTN_E_UNSUPPORTED, "P=%d exceeds ATTN_P_MAX=%d", P, ATTN_P_MAX);
  if (!o_partial || !lse_partial || !tickets) return fail(ATTN_E_WORKSPACE, "o_partial, lse_partial and tickets are required");
  if (!aligned(tickets, 4)) return fail(ATTN_E_ALIGN, "tickets must be 4-byte aligned");
  const int64_t RH = (int64_t)B * Nq * H;
  if (RH > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "B*Nq*H exceeds 2^31-1");
  if (RH * P > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "grid too large");
  rc = check_combine(o_partial, lse_partial, out, lse, P, B * Nq, H, D, dtype);
  if (rc) return rc;
  attn::DecodeParams p{};
  p.q = q; p.k = k; p.v = v; p.o_partial = o_partial; p.lse_partial = lse_partial; p.mask = mask;
  p.B = B; p.H = H; p.Nq = Nq; p.Nkv = Nkv; p.causal = causal; p.P = P;
  p.chunk = (int)(((int64_t)Nkv + P - 1) / P);
  p.scale_log2 = scale_log2(D);
  p.out = out; p.lse = lse; p.tickets = tickets;
  return hip_status(attn::launch_decode(p, dtype, D, true, (hipStream_t)stream), "attn_fwd_splitk_fused launch");
}

int attn_softmax_rows(const void* x, void* y, int64_t rows, int n, int dtype, int method, void* stream) {
  if (!x || !y) return fail(ATTN_E_NULL, "x and y must be non-NULL device pointers");
  if (rows < 1 || n < 1) return fail(ATTN_E_SHAPE, "rows and n must be >= 1 (got %lld, %d)", (long long)rows, n);
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16 && dtype != ATTN_FP32) return fail(ATTN_E_UNSUPPORTED, "dtype %d not supported", dtype);
  if (method != ATTN_SOFTMAX_STREAMING && method != ATTN_SOFTMAX_REGISTERS && method != ATTN_SOFTMAX_THREE_PASS)
    return fail(ATTN_E_UNSUPPORTED, "softmax method %d not supported", method);
  if (method == ATTN_SOFTMAX_REGISTERS && n > attn::softmax_regs_max_n())
    return fail(ATTN_E_UNSUPPORTED, "the registers method holds rows of at most %d elements (got %d)", attn::softmax_regs_max_n(), n);
  if ((rows + 3) / 4 > 0x7fffffffLL || (double)rows * n > 4.0e18) return fail(ATTN_E_SHAPE, "rows * n too large");
  if (method == ATTN_SOFTMAX_REGISTERS && n > 4096 && rows > 0x7fffffffLL) return fail(ATTN_E_SHAPE, "too many rows");
  const uintptr_t es = dtype == ATTN_FP32 ? 4 : 2;
  if (!aligned(x, es) || !aligned(y, es)) return fail(ATTN_E_ALIGN, "x and y must be aligned to their element size");
  const uintptr_t vb = 4 * es;   // four elements per vector access
  const bool vec = (n % 4 == 0) && aligned(x, vb) && aligned(y, vb);
  attn::SoftmaxParams p{x, y, rows, n};
  const int dt = dtype == ATTN_BF16 ? 0 : (dtype == ATTN_FP16 ? 1 : 2);
  return hip_status(attn::launch_softmax_rows(p, dt, method, vec, (hipStream_t)stream), "attn_softmax_rows launch");
}

int attn_round(const float* x, void* y, int64_t n, int dtype, void* stream) {
  if (n < 0) return fail(ATTN_E_SHAPE, "n must be >= 0 (got %lld)", (long long)n);
  if (n == 0) return ATTN_OK;
  if (!x || !y) return fail(ATTN_E_NULL, "x and y must be non-NULL device pointers");
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16 && dtype != ATTN_FP8_E4M3)
    return fail(ATTN_E_UNSUPPORTED, "dtype %d not supported (bf16, fp16 or E4M3)", dtype);
  if (!aligned(x, 4) || !aligned(y, dtype == ATTN_FP8_E4M3 ? 1 : 2)) return fail(ATTN_E_ALIGN, "x must be 4-byte and y element-size aligned");
  const int t = dtype == ATTN_BF16 ? 0 : (dtype == ATTN_FP16 ? 1 : 3);
  return hip_status(attn::launch_round(x, y, n, t, (hipStream_t)stream), "attn_round launch");
}

int attn_combine(const float* o_partial, const float* lse_partial, void* out, float* lse_out, int P,
                 int rows, int heads, int depth, int out_dtype, void* stream) {
  int rc = check_combine(o_partial, lse_partial, out, lse_out, P, rows, heads, depth, out_dtype);
  if (rc) return rc;
  return do_combine(o_partial, lse_partial, out, lse_out, P, rows, heads, depth, out_dtype, (hipStream_t)stream);
}

}  // extern "C"
