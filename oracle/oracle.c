/*
 * oracle.c -- plain, slow, FP64 CPU oracle for streaming online-softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library.  It shares no code, header, table or helper with the
 * HIP path, and the HIP path never calls it.
 *
 * Sources (web pages, cited by title and section):
 *   [TS]  Tylo.jl docs, "Streaming attention and online state": Online statistics;
 *         Same-lane conversion; Attention as a consumer.
 *   [TR]  Tylo.jl docs, "Register fragments and logical axes": Worked softmax;
 *         Logical types and register packing.
 *   [WS]  triton-cuda-lab workshop, "A3. Tiled attention with online normalization":
 *         Keep three quantities for each query row; Trace one query; Masks that preserve
 *         the recurrence.
 *   [SK]  Modular MAX Mojo module "fa4_splitk_combine": workspace layout and the per-row-head
 *         combine formulas.
 *
 * Everything is computed in double precision.  Inputs arrive as float32, bfloat16, float16,
 * 8-bit float (E4M3 / E5M2) or float64 element arrays and are widened to double exactly (every
 * such value is a double).
 *
 * Tensor layouts: q is [B, Nq, H, D]; k and v are [B, Nkv, H, D], D fastest.  A row-head index
 * rh = (b * Nq + i) * H + h names one query row of one head.  The optional mask is a row-major
 * [Nq, Nkv] byte array, nonzero = key visible, shared by every batch and head.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2, OR_E4M3 = 3, OR_E5M2 = 4, OR_F64 = 5 };
enum { OR_NO_NUMERATOR_RESCALE = 1, OR_SAME_BOUNDARY_BF16 = 2, OR_SAME_BOUNDARY_F16 = 4 };

/* ---------------------------------------------------------------------------------------------
 * Exact widening of stored elements to double.  bfloat16 is the top half of a float32;
 * float16 is decoded from its IEEE-754 binary16 fields (sign, 5-bit exponent, 10-bit fraction).
 * ------------------------------------------------------------------------------------------- */
static double decode_f16_bits(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double mag;
  if (e == 0) mag = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31) mag = f ? NAN : INFINITY;
  else mag = ldexp(1.0 + (double)f / 1024.0, e - 15);
  return sign ? -mag : mag;
}
static double decode_bf16_bits(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return (double)x;
}
/* 8-bit floats ([TR] Logical types and register packing: Float8E4M3, Float8E5M2), decoded from
 * their fields.  E4M3: sign, 4-bit exponent (bias 7), 3-bit fraction; exponent 0 is subnormal
 * (f * 2^-9); there are no infinities and S.1111.111 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448.  E5M2: sign, 5-bit exponent (bias 15), 2-bit fraction, IEEE-like (exponent 0
 * subnormal f * 2^-16; exponent 31: infinity if f = 0, else NaN). */
static double decode_e4m3_bits(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 15, f = c & 7;
  double mag;
  if (e == 15 && f == 7) mag = NAN;
  else if (e == 0) mag = ldexp((double)f, -9);
  else mag = ldexp(1.0 + f / 8.0, e - 7);
  return sign ? -mag : mag;
}
static double decode_e5m2_bits(uint8_t c) {
  int sign = c >> 7, e = (c >> 2) & 31, f = c & 3;
  double mag;
  if (e == 31) mag = f ? NAN : INFINITY;
  else if (e == 0) mag = ldexp((double)f, -16);
  else mag = ldexp(1.0 + f / 4.0, e - 15);
  return sign ? -mag : mag;
}
static double load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == OR_F32) return (double)((const float*)base)[idx];
  if (dtype == OR_F64) return ((const double*)base)[idx];
  if (dtype == OR_E4M3) return decode_e4m3_bits(((const uint8_t*)base)[idx]);
  if (dtype == OR_E5M2) return decode_e5m2_bits(((const uint8_t*)base)[idx]);
  uint16_t bits = ((const uint16_t*)base)[idx];
  return dtype == OR_BF16 ? decode_bf16_bits(bits) : decode_f16_bits(bits);
}

void oracle_decode(const void* src, int dtype, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, i, dtype);
}

/* ---------------------------------------------------------------------------------------------
 * O4. Round-to-nearest-even conversion of a float32 to bfloat16 / float16 bits, written from the
 * definition rather than from bit manipulation: list the two neighbouring representable values
 * (exact in double), take the nearer, and on a tie the one whose last significand bit is even.
 * Signed zeros and infinities map to themselves, NaN maps to a NaN, there is no saturation to
 * the largest finite value and no flush of subnormals ([TS] Same-lane conversion, last
 * paragraph; [TR] Logical types and register packing).
 *
 * A format is (p = significand bits incl. the implicit one, emin = exponent of the smallest
 * normal, emax = exponent of the largest finite value, ebits).
 * ------------------------------------------------------------------------------------------- */
typedef struct { int p, emin, emax, ebits; } fmt_t;
static const fmt_t FMT_BF16 = {8, -126, 127, 8};
static const fmt_t FMT_F16 = {11, -14, 15, 5};

static uint16_t encode_small(double mag, int sign, fmt_t f) {
  /* mag is exactly representable in f (or +inf). */
  int mbits = f.p - 1, bias = (1 << (f.ebits - 1)) - 1;
  uint32_t e_field, m_field;
  if (isinf(mag)) { e_field = (1u << f.ebits) - 1; m_field = 0; }
  else if (mag == 0.0) { e_field = 0; m_field = 0; }
  else {
    int e;
    frexp(mag, &e);      /* mag = fr * 2^e, fr in [0.5, 1) -> unbiased exponent e-1 */
    int E = e - 1;
    if (E < f.emin) {    /* subnormal: mag = m * 2^(emin - mbits) */
      e_field = 0;
      m_field = (uint32_t)ldexp(mag, -(f.emin - mbits));
    } else {
      e_field = (uint32_t)(E + bias);
      m_field = (uint32_t)(ldexp(mag, -E) * (double)(1u << mbits)) - (1u << mbits);
    }
  }
  return (uint16_t)((sign << 15) | (e_field << mbits) | m_field);
}

static uint16_t round_rne(float xf, fmt_t f) {
  double x = (double)xf;
  int sign = signbit(x) ? 1 : 0;
  if (isnan(x)) return (uint16_t)(0x7fff);            /* some quiet NaN (all ones) */
  double a = fabs(x);
  if (isinf(a) || a == 0.0) return encode_small(a, sign, f);
  /* spacing of representable values around a */
  int e;
  frexp(a, &e);
  int E = e - 1;
  if (E < f.emin) E = f.emin;
  double ulp = ldexp(1.0, E - (f.p - 1));
  double lo = floor(a / ulp) * ulp;                   /* exact: a/ulp is exact (power of two) */
  double hi = lo + ulp;
  double pick;
  if (a - lo < hi - a) pick = lo;
  else if (hi - a < a - lo) pick = hi;
  else pick = (fmod(lo / ulp, 2.0) == 0.0) ? lo : hi; /* tie: even last significand bit */
  double maxfin = ldexp(2.0 - ldexp(1.0, -(f.p - 1)), f.emax);
  if (pick > maxfin) pick = INFINITY;                 /* no saturation */
  return encode_small(pick, sign, f);
}

uint16_t oracle_round_bf16(float x) { return round_rne(x, FMT_BF16); }
uint16_t oracle_round_f16(float x) { return round_rne(x, FMT_F16); }

void oracle_round_array(const float* x, int64_t n, int target_dtype, uint16_t* out) {
  fmt_t f = target_dtype == OR_BF16 ? FMT_BF16 : FMT_F16;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = round_rne(x[i], f);
}

/* ---------------------------------------------------------------------------------------------
 * O6. Round-to-nearest-even conversion of a float32 to E4M3 / E5M2 bits with saturation to the
 * largest finite value ([TR] Logical types and register packing: FP32 values are converted to the
 * two 8-bit formats by nearest-even rounding, and magnitudes past the format's range are clamped
 * to its largest finite value rather than becoming infinite).  Same construction as
 * O4: the two neighbouring values at the input's binade spacing (exponent range unbounded
 * above), the nearer, ties to the even last significand bit; a result beyond the largest finite
 * value (448 for E4M3, 57344 for E5M2), and an infinite input, become that value with the
 * input's sign.  Signed zeros are kept, subnormals are not flushed, NaN gives a NaN.
 * ------------------------------------------------------------------------------------------- */
typedef struct { int p, emin, ebits; double maxfin; } fmt8_t;
static const fmt8_t FMT_E4M3 = {4, -6, 4, 448.0};
static const fmt8_t FMT_E5M2 = {3, -14, 5, 57344.0};

static uint8_t encode8(double mag, int sign, fmt8_t f) {
  /* mag is finite and exactly representable in f */
  int mbits = f.p - 1, bias = (1 << (f.ebits - 1)) - 1;
  uint32_t e_field = 0, m_field = 0;
  if (mag != 0.0) {
    int e;
    frexp(mag, &e);
    int E = e - 1;
    if (E < f.emin) {
      m_field = (uint32_t)ldexp(mag, -(f.emin - mbits));
    } else {
      e_field = (uint32_t)(E + bias);
      m_field = (uint32_t)(ldexp(mag, -E) * (double)(1u << mbits)) - (1u << mbits);
    }
  }
  return (uint8_t)((sign << 7) | (e_field << mbits) | m_field);
}

static uint8_t round_fp8(float xf, fmt8_t f) {
  double x = (double)xf;
  int sign = signbit(x) ? 1 : 0;
  if (isnan(x)) return (uint8_t)0x7f;                 /* a NaN in both formats */
  double a = fabs(x);
  if (isinf(a)) return encode8(f.maxfin, sign, f);
  if (a == 0.0) return (uint8_t)(sign << 7);
  int e;
  frexp(a, &e);
  int E = e - 1;
  if (E < f.emin) E = f.emin;
  double ulp = ldexp(1.0, E - (f.p - 1));
  double lo = floor(a / ulp) * ulp;
  double hi = lo + ulp;
  double pick;
  if (a - lo < hi - a) pick = lo;
  else if (hi - a < a - lo) pick = hi;
  else pick = (fmod(lo / ulp, 2.0) == 0.0) ? lo : hi;
  if (pick > f.maxfin) pick = f.maxfin;               /* saturate to finite */
  return encode8(pick, sign, f);
}

void oracle_round_fp8_array(const float* x, int64_t n, int target_dtype, uint8_t* out) {
  fmt8_t f = target_dtype == OR_E4M3 ? FMT_E4M3 : FMT_E5M2;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = round_fp8(x[i], f);
}

/* Same-boundary rounding of a weight: the caller passes the weight already rounded to float32
 * (the precision in which a kernel holds it); this rounds that float32 to bf16 / f16 and widens
 * the result back to double. */
static double round_value(float x, int flags) {
  uint16_t bits = (flags & OR_SAME_BOUNDARY_BF16) ? oracle_round_bf16(x) : oracle_round_f16(x);
  return (flags & OR_SAME_BOUNDARY_BF16) ? decode_bf16_bits(bits) : decode_f16_bits(bits);
}

/* ---------------------------------------------------------------------------------------------
 * Visibility of key j to query i ([WS] Masks that preserve the recurrence: causal includes the
 * diagonal; [TS] Attention as a consumer: optional Boolean M x N mask; a key index past the
 * key length is never visible).
 * ------------------------------------------------------------------------------------------- */
static int visible(int i, int j, int Nkv, int causal, const uint8_t* mask) {
  if (j >= Nkv) return 0;
  if (causal && j > i) return 0;
  if (mask && mask[(int64_t)i * Nkv + j] == 0) return 0;
  return 1;
}

static int64_t qk_index(int b, int t, int h, int N, int H, int D) {
  return (((int64_t)b * N + t) * H + h) * D;
}

/* scaled logit s_ij = (q_i . k_j) / sqrt(D)  ([WS] Keep three quantities for each query row) */
static double logit(const void* q, const void* k, int dt, int b, int i, int j, int h, int Nq, int Nkv,
                    int H, int D) {
  int64_t qo = qk_index(b, i, h, Nq, H, D), ko = qk_index(b, j, h, Nkv, H, D);
  double acc = 0.0;
  for (int d = 0; d < D; ++d) acc += load_elem(q, qo + d, dt) * load_elem(k, ko + d, dt);
  return acc / sqrt((double)D);
}

static void rh_split(int64_t rh, int Nq, int H, int* b, int* i, int* h) {
  *h = (int)(rh % H);
  int64_t t = rh / H;
  *i = (int)(t % Nq);
  *b = (int)(t / Nq);
}

/* ---------------------------------------------------------------------------------------------
 * O1. Dense definition of attention for the selected row-heads.
 *   vis(i) = visible keys.  If vis(i) is empty: O_i = 0, LSE_i = -inf ([TS] Online statistics and
 *   [TR] Worked softmax: a row with every key masked yields zeros and a log-sum-exp of -inf).
 *   Otherwise M = max_j s_ij, w_j = exp(s_ij - M), L = sum w_j, O_i = sum_j w_j v_j / L and
 *   LSE_i = M + ln L (natural log).
 * sel: row-head indices (NULL = all B*Nq*H in order).  out: [nsel, D]; lse: [nsel] (nullable).
 * ------------------------------------------------------------------------------------------- */
int oracle_attn_dense(const void* q, const void* k, const void* v, int dt, const uint8_t* mask,
                      int B, int H, int Nq, int Nkv, int D, int causal, const int64_t* sel,
                      int64_t nsel, double* out, double* lse) {
  if (!sel) nsel = (int64_t)B * Nq * H;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nsel; ++r) {
    int64_t rh = sel ? sel[r] : r;
    int b, i, h;
    rh_split(rh, Nq, H, &b, &i, &h);
    double* s = (double*)malloc(sizeof(double) * (Nkv > 0 ? Nkv : 1));
    if (!s) { err = 1; continue; }
    double* o = out + r * D;
    int any = 0;
    double M = -INFINITY;
    for (int j = 0; j < Nkv; ++j) {
      if (!visible(i, j, Nkv, causal, mask)) continue;
      s[j] = logit(q, k, dt, b, i, j, h, Nq, Nkv, H, D);
      if (!any || s[j] > M) M = s[j];
      any = 1;
    }
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (!any) {
      if (lse) lse[r] = -INFINITY;
      free(s);
      continue;
    }
    double L = 0.0;
    for (int j = 0; j < Nkv; ++j) {
      if (!visible(i, j, Nkv, causal, mask)) continue;
      double w = exp(s[j] - M);
      L += w;
      int64_t vo = qk_index(b, j, h, Nkv, H, D);
      for (int d = 0; d < D; ++d) o[d] += w * load_elem(v, vo + d, dt);
    }
    for (int d = 0; d < D; ++d) o[d] /= L;
    if (lse) lse[r] = M + log(L);
    free(s);
  }
  return err;
}

/* ---------------------------------------------------------------------------------------------
 * O2. The online recurrence over BN-key tiles ([WS] Keep three quantities for each query row;
 * [TS] Online statistics for the empty state and the guards; [TR] Worked softmax).
 *
 * A query row carries a summary of the keys absorbed so far: the reference m (their largest
 * logit, -inf before any visible key), l (the sum of their exponentials taken against m) and
 * a[D] (the same exponentials weighting their value rows).  A tile is absorbed in the order the
 * workshop gives: the reference moves to the larger of m and the tile's largest logit; the old
 * l and a, expressed against the old reference, shrink by exp(old - new) (0 for the empty
 * summary); the tile's exponentials against the new reference are added to l, and their
 * value-weighted sums to a.  While the reference is still -inf the exponentials are taken
 * against 0, so no -inf - (-inf) arises and a masked logit (-inf) weighs exactly 0.  Finally
 * O = a / l and LSE = m + ln l, or 0 and -inf when nothing was visible (l = 0).
 *
 * flags: OR_NO_NUMERATOR_RESCALE keeps a unshrunk when the reference moves (the mistake the
 * worked trace exposes, which turns its 6 into 7); OR_SAME_BOUNDARY_* rounds each weight to bf16
 * / f16 before it multiplies its value row, while l takes the weight unrounded ([TS] Attention as
 * a consumer).  tile_trace (nullable) receives (m, l, a[0], shrink factor) after every tile.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
  double m;    /* reference: the largest logit absorbed (-inf: none visible yet) */
  double l;    /* sum over absorbed keys of exp(logit - m) */
  double* a;   /* sum over absorbed keys of exp(logit - m) * value row (D entries) */
} row_state_t;

/* Absorbs keys j0 .. j1-1 (logits s, value rows vrows[j*D ..]) into st; w holds j1 - j0 doubles
 * of scratch.  Returns the factor the previous l and a were scaled by. */
static double absorb_tile(row_state_t* st, const double* s, const double* vrows, int j0, int j1, int D,
                          int flags, double* w) {
  double ref = st->m;
  for (int j = j0; j < j1; ++j)
    if (s[j] > ref) ref = s[j];
  const double base = (ref == -INFINITY) ? 0.0 : ref;
  const double shrink = exp(st->m - base);
  double tile_l = 0.0;
  for (int j = j0; j < j1; ++j) {
    w[j - j0] = exp(s[j] - base);
    tile_l += w[j - j0];
  }
  st->l = shrink * st->l + tile_l;
  const double keep = (flags & OR_NO_NUMERATOR_RESCALE) ? 1.0 : shrink;
  const int rounded = flags & (OR_SAME_BOUNDARY_BF16 | OR_SAME_BOUNDARY_F16);
  for (int d = 0; d < D; ++d) {
    double acc = keep * st->a[d];
    for (int j = j0; j < j1; ++j) {
      const double wj = rounded ? round_value((float)w[j - j0], flags) : w[j - j0];
      acc += wj * vrows[(int64_t)j * D + d];
    }
    st->a[d] = acc;
  }
  st->m = ref;
  return shrink;
}

static void online_core(const double* s, const double* vrows, int n, int D, int BN, int flags,
                        double* o, double* lse, double* tile_trace) {
  row_state_t st = {-INFINITY, 0.0, (double*)calloc((size_t)(D > 0 ? D : 1), sizeof(double))};
  double* w = (double*)malloc(sizeof(double) * (size_t)(BN > 0 ? BN : 1));
  int tile = 0;
  for (int j0 = 0; j0 < n; j0 += BN, ++tile) {
    const double shrink = absorb_tile(&st, s, vrows, j0, j0 + BN < n ? j0 + BN : n, D, flags, w);
    if (tile_trace) {
      double* t = tile_trace + 4 * tile;
      t[0] = st.m;
      t[1] = st.l;
      t[2] = st.a[0];
      t[3] = shrink;
    }
  }
  const int seen = st.l != 0.0;
  for (int d = 0; d < D; ++d) o[d] = seen ? st.a[d] / st.l : 0.0;
  if (lse) *lse = seen ? st.m + log(st.l) : -INFINITY;
  free(w);
  free(st.a);
}

/* Logits-in entry point for the worked trace: s[n] are already-scaled logits (-inf = masked),
 * v[n][D] the value rows. */
void oracle_online_from_logits(const double* s, const double* v, int n, int D, int BN, int flags,
                               double* out, double* lse, double* tile_trace) {
  online_core(s, v, n, D, BN, flags, out, lse, tile_trace);
}

int oracle_attn_online(const void* q, const void* k, const void* v, int dt, const uint8_t* mask,
                       int B, int H, int Nq, int Nkv, int D, int causal, int BN, int flags,
                       const int64_t* sel, int64_t nsel, double* out, double* lse) {
  if (!sel) nsel = (int64_t)B * Nq * H;
  if (BN < 1) return 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nsel; ++r) {
    int64_t rh = sel ? sel[r] : r;
    int b, i, h;
    rh_split(rh, Nq, H, &b, &i, &h);
    double* s = (double*)malloc(sizeof(double) * (Nkv > 0 ? Nkv : 1));
    double* vr = (double*)malloc(sizeof(double) * ((int64_t)(Nkv > 0 ? Nkv : 1) * D));
    for (int j = 0; j < Nkv; ++j) {
      s[j] = visible(i, j, Nkv, causal, mask) ? logit(q, k, dt, b, i, j, h, Nq, Nkv, H, D) : -INFINITY;
      int64_t vo = qk_index(b, j, h, Nkv, H, D);
      for (int d = 0; d < D; ++d) vr[(int64_t)j * D + d] = load_elem(v, vo + d, dt);
    }
    online_core(s, vr, Nkv, D, BN, flags, out + r * D, lse ? lse + r : NULL, NULL);
    free(s);
    free(vr);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * O3a. softmax_merge of two independent summaries (m, l, a) ([TS] Online statistics: the merge
 * of two summaries, returning the rescale factor of each numerator):
 *   m = max(m1, m2); alpha_k = exp(m_k - m) (0 for an empty summary);
 *   l = alpha1 l1 + alpha2 l2;  a = alpha1 a1 + alpha2 a2.  Two empty inputs give an empty result.
 * ------------------------------------------------------------------------------------------- */
void oracle_merge_nat(double m1, double l1, const double* a1, double m2, double l2, const double* a2,
                      int D, double* m, double* l, double* a, double* alpha1, double* alpha2) {
  double mm = m1 > m2 ? m1 : m2;
  double al1 = (m1 == -INFINITY) ? 0.0 : exp(m1 - mm);
  double al2 = (m2 == -INFINITY) ? 0.0 : exp(m2 - mm);
  *m = mm;
  *l = al1 * l1 + al2 * l2;
  for (int d = 0; d < D; ++d) a[d] = al1 * a1[d] + al2 * a2[d];
  *alpha1 = al1;
  *alpha2 = al2;
}

/* ---------------------------------------------------------------------------------------------
 * O3b. The LSE-weighted combine of a split-K workspace, base 2 throughout ([SK] per-row-head
 * formulas): for each row-head, m* = max_p lse_p; G = log2(sum_p 2^(lse_p - m*)) + m*;
 * scale_p = 2^(lse_p - G); O[d] = sum_p scale_p * o_partial[p, rh, d].  A partition with
 * lse_p = -inf gets scale 0; when every partition is empty the output is 0 and G = -inf (the
 * all-masked convention of [TR] Worked softmax applied to the combine).
 * o_partial: [P, RH, D]; lse_partial: [P, RH]; out: [RH, D]; g_out (nullable): [RH], base 2.
 * ------------------------------------------------------------------------------------------- */
void oracle_combine_log2(const double* o_partial, const double* lse_partial, int P, int64_t RH, int D,
                         double* out, double* g_out) {
#pragma omp parallel for schedule(static)
  for (int64_t rh = 0; rh < RH; ++rh) {
    double ms = -INFINITY;
    for (int p = 0; p < P; ++p) if (lse_partial[(int64_t)p * RH + rh] > ms) ms = lse_partial[(int64_t)p * RH + rh];
    double* o = out + rh * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (ms == -INFINITY) {
      if (g_out) g_out[rh] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int p = 0; p < P; ++p) {
      double lp = lse_partial[(int64_t)p * RH + rh];
      sum += (lp == -INFINITY) ? 0.0 : exp2(lp - ms);
    }
    double G = log2(sum) + ms;
    for (int p = 0; p < P; ++p) {
      double lp = lse_partial[(int64_t)p * RH + rh];
      double sc = (lp == -INFINITY) ? 0.0 : exp2(lp - G);
      const double* op = o_partial + ((int64_t)p * RH + rh) * D;
      for (int d = 0; d < D; ++d) o[d] += sc * op[d];
    }
    if (g_out) g_out[rh] = G;
  }
}

/* ---------------------------------------------------------------------------------------------
 * O3c. The split-K producer's workspace ([SK] workspace layout): key partition p covers
 * [p*c, min((p+1)*c, Nkv)) with c = ceil(Nkv / P).  For each partition, the dense definition
 * restricted to the partition's visible keys gives the locally normalised O_p / l_p and
 * lse_p = log2 of the partition's sum of exponentials = (M + ln L) / ln 2.  An empty partition
 * gives o_partial = 0 and lse_partial = -inf.
 * o_partial: [P, nsel, D]; lse_partial: [P, nsel] (base 2).
 * ------------------------------------------------------------------------------------------- */
int oracle_splitk(const void* q, const void* k, const void* v, int dt, const uint8_t* mask, int B,
                  int H, int Nq, int Nkv, int D, int causal, int P, const int64_t* sel, int64_t nsel,
                  double* o_partial, double* lse_partial) {
  if (!sel) nsel = (int64_t)B * Nq * H;
  if (P < 1) return 1;
  int64_t c = ((int64_t)Nkv + P - 1) / P;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int p = 0; p < P; ++p) {
    for (int64_t r = 0; r < nsel; ++r) {
      int64_t rh = sel ? sel[r] : r;
      int b, i, h;
      rh_split(rh, Nq, H, &b, &i, &h);
      int64_t j0 = (int64_t)p * c, j1 = j0 + c < Nkv ? j0 + c : Nkv;
      double* o = o_partial + ((int64_t)p * nsel + r) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      double M = -INFINITY;
      int any = 0;
      for (int64_t j = j0; j < j1; ++j) {
        if (!visible(i, (int)j, Nkv, causal, mask)) continue;
        double s = logit(q, k, dt, b, i, (int)j, h, Nq, Nkv, H, D);
        if (!any || s > M) M = s;
        any = 1;
      }
      if (!any) {
        lse_partial[(int64_t)p * nsel + r] = -INFINITY;
        continue;
      }
      double L = 0.0;
      for (int64_t j = j0; j < j1; ++j) {
        if (!visible(i, (int)j, Nkv, causal, mask)) continue;
        double w = exp(logit(q, k, dt, b, i, (int)j, h, Nq, Nkv, H, D) - M);
        L += w;
        int64_t vo = qk_index(b, (int)j, h, Nkv, H, D);
        for (int d = 0; d < D; ++d) o[d] += w * load_elem(v, vo + d, dt);
      }
      for (int d = 0; d < D; ++d) o[d] /= L;
      lse_partial[(int64_t)p * nsel + r] = (M + log(L)) / log(2.0);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------
 * O5. Row softmax with the all-masked convention ([TR] "Worked softmax"; [TS] Online statistics):
 * for each row of n logits, y_j = exp(x_j - M) / sum_k exp(x_k - M) with M the row maximum.  A
 * logit of -inf is a masked entry and gets weight 0.  A row whose entries are all -inf has no
 * finite maximum; subtracting it would give -inf - (-inf), so such a row is defined as all zeros
 * and handled before any subtraction.  Otherwise the entry equal to M contributes exp(0) = 1, so
 * the sum is at least 1 and the division is safe.  x is a row-major [rows, n] array of float32,
 * bfloat16 or float16; y is [rows, n] double.
 * ------------------------------------------------------------------------------------------- */
void oracle_softmax_rows(const void* x, int dtype, int64_t rows, int64_t n, double* y) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < rows; ++r) {
    double* yr = y + r * n;
    double top = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
      const double v = load_elem(x, r * n + j, dtype);
      if (v > top) top = v;
    }
    if (top == -INFINITY) {                 /* every entry masked */
      for (int64_t j = 0; j < n; ++j) yr[j] = 0.0;
      continue;
    }
    double total = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      yr[j] = exp(load_elem(x, r * n + j, dtype) - top);   /* -inf entries give 0 */
      total += yr[j];
    }
    for (int64_t j = 0; j < n; ++j) yr[j] /= total;
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
