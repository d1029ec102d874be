/*
 * oracle.c -- plain, slow, scalar CPU oracle for asymmetric low-bit KV-cache
 * quantization and single-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the HIP library.
 *
 * What it computes, and the passage each step follows (pages are cited by
 * title and section):
 *
 *  - Keys are quantized per channel (statistics gathered along tokens), values
 *    per token (statistics gathered along channels), and the most recent
 *    tokens stay in an unquantized fp16 window: "[Framework] The Asymmetric
 *    Key-Value Cache Compression", section III (KIVI partitioning: the
 *    per-channel / per-token split and the FP16 sliding window of recent
 *    tokens); "Asymmetric Key-Value Quantization: 2-Bit Values and 4-Bit Keys
 *    under Long-Context Drift", section 3.1 (bit-width allocation, K4/V2).
 *  - The quantizer is the textbook asymmetric (affine, min/max) uniform
 *    quantizer.  The pages call the scheme asymmetric and tuning-free but
 *    print no formula; this is the plainest reading (scale = range/(2^b-1),
 *    zero point = group minimum, code = round-half-even((x-min)/scale)).
 *  - Optional key rotation by the normalized Walsh-Hadamard transform,
 *    computed with the O(N log N) butterfly: "[Framework] ...", section IV
 *    (stage 1, canalized rotation Y = X H).
 *  - Attention is softmax(q K^T / sqrt(d)) V: "Asymmetric Key-Value
 *    Quantization ...", section 1, evaluated in fp64 on the decoded cache.
 *  - Attention-sink window: the first S0 tokens stay in fp16 next to the
 *    window of recent tokens ("[Framework] ...", section IV, on the initial
 *    attention-sink tokens; the high-precision windows for recent and sink
 *    tokens of the InnerQ abstract on the page "WUSH-KV: KV Cache
 *    Quantization with Data-Adaptive Transforms").  Quantized groups start
 *    at token S0.
 *  - Hybrid quantization: per group, a symmetric or the asymmetric quantizer,
 *    chosen from the group's own values (InnerQ abstract, same page).  The
 *    page names no symmetric formula and no selection rule; here symmetric is
 *    x = s (code - c0), c0 = 2^(b-1) - 1, s = max|x| / c0, and the quantizer
 *    with the smaller largest reconstruction error on the group is kept.
 *  - Token-norm scaling of the rotated keys (OScaR stage 2: "[Framework]
 *    ...", section IV, omni-token scaling): each quantized key token is
 *    divided by its L2 norm before the per-channel quantizer, and the norm is
 *    kept (fp16) and multiplied back at decode.  The page gives no arithmetic;
 *    here the norm is that of the fp16 (rotated) token row, summed as a fixed
 *    pairwise tree in binary32 with a correctly rounded square root, the
 *    normalized values are rounded to fp16, and a zero row keeps norm 0.
 *  - Position-adaptive bit widths ("Asymmetric Key-Value Quantization ...",
 *    section 3.2: high bits for the most recent Delta tokens, low bits for the
 *    first Delta, middle bits between; section 7 notes that the method needs
 *    token positions when it quantizes).  Here a group's bits are fixed when
 *    it is quantized, from the sequence length n after the append that
 *    quantizes it: recent if its last token is among the last Delta of n,
 *    otherwise early if its last token is among the first Delta, otherwise
 *    middle (the printed cases, recent taking precedence where they overlap).
 *  - Drift detection ("Asymmetric Key-Value Quantization ...", section 3.3:
 *    the KL divergence of the current distribution of quantized values from
 *    the calibration distribution, a threshold of 0.1 triggering a
 *    requantization of the affected tokens).  Here the distributions are code
 *    histograms: a group's key codes (all G x D of them) and value codes,
 *    against the pooled code histogram of a calibration range of groups of
 *    the same kv head; KL in natural log with 0 log 0 = 0 and +inf where the
 *    calibration has no mass; a group is flagged when its KL exceeds the
 *    threshold.  The requantization itself is the uniform quantizer applied
 *    again to the affected groups' tokens (the page's Lloyd-Max step is not
 *    reproduced), i.e. the ordinary encoding of those tokens.
 *  - Bits-per-element accounting: "Asymmetric Key-Value Quantization ...",
 *    section 3.1 (average of key and value bit widths) and section 3.4
 *    (combined compression table); here the per-group fp16 scale and zero
 *    and the fp16 window are counted as well.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64 SSE arithmetic is IEEE binary32/binary64 with round-to-nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

int64_t orc_encode_slice_ext(const void* k, const void* v, int dtype, int64_t n, int D,
                             int kbits, int vbits, int G, int R, int rotate, int S0, int hybrid,
                             int token_norm, uint16_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                             uint16_t* v_codes, uint16_t* v_scale, uint16_t* v_zero,
                             uint16_t* k_resid, uint16_t* v_resid, uint8_t* k_sym, uint8_t* v_sym,
                             uint16_t* k_norm, const uint8_t* group_kbits, const uint8_t* group_vbits);
double orc_bits_per_element_sink(int64_t n, int kbits, int vbits, int G, int R, int S0,
                                 double overhead_bits);

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 and bfloat16 conversions, written from the formats.     */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t orc_f32_to_f16(float x) {
  uint32_t u = f32_bits(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t ax = u & 0x7fffffffu;
  if (ax > 0x7f800000u) /* NaN: keep a quiet NaN with the top payload bits */
    return (uint16_t)(sign | 0x7e00u | ((ax >> 13) & 0x1ffu));
  if (ax >= 0x477ff000u) /* >= 65520 rounds to infinity (65520 is a tie, 65504 is odd) */
    return (uint16_t)(sign | 0x7c00u);
  if (ax >= 0x38800000u) { /* normal binary16 result: |x| >= 2^-14 */
    uint32_t e = (ax >> 23) - 127u + 15u;
    uint32_t mant = ax & 0x7fffffu;
    uint32_t h = (e << 10) | (mant >> 13);
    uint32_t rem = mant & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* carry may bump the exponent: correct */
    return (uint16_t)(sign | h);
  }
  if (ax <= 0x33000000u) /* |x| <= 2^-25: rounds to zero (2^-25 is a tie to even 0) */
    return sign;
  { /* subnormal binary16 result: value = round(|x| * 2^24) units of 2^-24 */
    int e = (int)(ax >> 23) - 127;          /* -25 < e < -14 */
    uint32_t m = (ax & 0x7fffffu) | 0x800000u; /* |x| = m * 2^(e-23) */
    int shift = -e - 1;                      /* |x| * 2^24 = m >> shift */
    uint32_t q = m >> shift;
    uint32_t rem = m & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    return (uint16_t)(sign | q);
  }
}

float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1fu;
  uint32_t m = h & 0x3ffu;
  if (e == 0x1f) return bits_f32(sign | 0x7f800000u | (m << 13));
  if (e == 0) {
    /* zero or subnormal: m * 2^-24, exact in binary32 */
    float v = (float)m * 5.9604644775390625e-08f;
    return sign ? -v : v;
  }
  return bits_f32(sign | ((e - 15u + 127u) << 23) | (m << 13));
}

float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even (used by the pins). */
uint16_t orc_f32_to_bf16(float x) {
  uint32_t u = f32_bits(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* Widen one stored input element of the given dtype to binary32 (exact). */
static float load_in(const void* p, int dtype, size_t i) {
  if (dtype == ORC_F32) return ((const float*)p)[i];
  if (dtype == ORC_F16) return orc_f16_to_f32(((const uint16_t*)p)[i]);
  return orc_bf16_to_f32(((const uint16_t*)p)[i]);
}

/* ------------------------------------------------------------------------ */
/* Walsh-Hadamard rotation ("[Framework] ...", section IV, stage 1).         */
/* ------------------------------------------------------------------------ */

/* In place, n a power of two: unnormalized butterflies in Sylvester
 * (natural) order with span h = 1, 2, 4, ..., n/2, each pair (a, b) becoming
 * (a + b, a - b) in binary32, then one multiply of every element by the
 * binary32 value nearest to 1/sqrt(n). */
void orc_fwht_f32(float* y, int n) {
  for (int h = 1; h < n; h <<= 1)
    for (int i = 0; i < n; ++i)
      if ((i & h) == 0) {
        float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  float c = (float)(1.0 / sqrt((double)n));
  for (int i = 0; i < n; ++i) y[i] = y[i] * c;
}

/* Rotate a query by the exact normalized Sylvester matrix in fp64:
 * out_j = sum_i q_i H_ij / sqrt(n), H_ij = (-1)^popcount(i & j). */
void orc_rotate_f64(const double* q, double* out, int n) {
  double inv = 1.0 / sqrt((double)n);
  for (int j = 0; j < n; ++j) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += (__builtin_popcount((unsigned)(i & j)) & 1) ? -q[i] : q[i];
    out[j] = s * inv;
  }
}

/* ------------------------------------------------------------------------ */
/* Asymmetric uniform quantizer for one group.                               */
/* ------------------------------------------------------------------------ */

/* x: `count` values, each already an fp16 value widened to binary32.
 * Outputs: codes[count] in [0, 2^bits - 1]; the binary32 scale and minimum
 * actually used for the codes; their fp16 storage forms.
 *   mn = min x, mx = max x (both + 0.0f, so -0 becomes +0)
 *   s  = (mx - mn) / (2^bits - 1), IEEE binary32 division
 *   code = clamp(rne((x - mn) / s), 0, 2^bits - 1), or 0 for every x if s == 0
 *   scale16 = fp16_rne(s), zero16 = fp16(mn) (exact: mn is an fp16 value) */
void orc_quantize_group(const float* x, int count, int bits, uint16_t* codes,
                        float* s_out, float* mn_out, uint16_t* scale16, uint16_t* zero16) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < count; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  float levels = (float)((1u << bits) - 1u);
  float s = (mx - mn) / levels;
  for (int i = 0; i < count; ++i) {
    if (s == 0.0f) { codes[i] = 0; continue; }
    float q = rintf((x[i] - mn) / s);
    if (q < 0.0f) q = 0.0f;
    if (q > levels) q = levels;
    codes[i] = (uint16_t)q;
  }
  if (s_out) *s_out = s;
  if (mn_out) *mn_out = mn;
  *scale16 = orc_f32_to_f16(s);
  *zero16 = orc_f32_to_f16(mn);
}

/* Symmetric uniform quantizer for one group (same inputs as above), levels
 * c0 = 2^(bits-1) - 1 on either side of zero:
 *   M  = max |x| (+ 0.0f), s = M / c0, IEEE binary32 division
 *   code = clamp(rne(x / s), -c0, c0) + c0, or c0 for every x if s == 0
 *   scale16 = fp16_rne(s), zero16 = fp16_rne(-(scale16 * c0))
 * so that zero16 + code * scale16 reconstructs s16 * (code - c0) up to the
 * rounding of zero16. */
void orc_quantize_group_sym(const float* x, int count, int bits, uint16_t* codes, float* s_out,
                            uint16_t* scale16, uint16_t* zero16) {
  float M = 0.0f;
  for (int i = 0; i < count; ++i) {
    float a = fabsf(x[i]);
    if (a > M) M = a;
  }
  M = M + 0.0f;
  float c0 = (float)((1u << (bits - 1)) - 1u);
  float s = M / c0;
  for (int i = 0; i < count; ++i) {
    if (s == 0.0f) { codes[i] = (uint16_t)c0; continue; }
    float q = rintf(x[i] / s);
    if (q < -c0) q = -c0;
    if (q > c0) q = c0;
    codes[i] = (uint16_t)(q + c0);
  }
  if (s_out) *s_out = s;
  *scale16 = orc_f32_to_f16(s);
  *zero16 = orc_f32_to_f16(-(orc_f16_to_f32(*scale16) * c0));
}

/* Largest reconstruction error of a group in binary32: for each x,
 * xhat = fp32(code * scale16) + zero16 (the product is exact, the sum is
 * rounded), e = |x - xhat| (rounded); the maximum is exact. */
float orc_group_max_error(const float* x, const uint16_t* codes, int count, uint16_t scale16,
                          uint16_t zero16) {
  float s = orc_f16_to_f32(scale16), z = orc_f16_to_f32(zero16), E = 0.0f;
  for (int i = 0; i < count; ++i) {
    float xh = (float)codes[i] * s;
    xh = xh + z;
    float e = fabsf(x[i] - xh);
    if (e > E) E = e;
  }
  return E;
}

/* Hybrid: both quantizers, keep the symmetric one only if its largest error
 * is strictly smaller.  Returns 1 if the symmetric quantizer was kept. */
int orc_quantize_group_hybrid(const float* x, int count, int bits, uint16_t* codes,
                              uint16_t* scale16, uint16_t* zero16) {
  uint16_t* cs = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)count);
  uint16_t sa, za, ss, zs;
  orc_quantize_group(x, count, bits, codes, NULL, NULL, &sa, &za);
  orc_quantize_group_sym(x, count, bits, cs, NULL, &ss, &zs);
  float ea = orc_group_max_error(x, codes, count, sa, za);
  float es = orc_group_max_error(x, cs, count, ss, zs);
  int sym = es < ea;
  if (sym) {
    memcpy(codes, cs, sizeof(uint16_t) * (size_t)count);
    *scale16 = ss;
    *zero16 = zs;
  } else {
    *scale16 = sa;
    *zero16 = za;
  }
  free(cs);
  return sym;
}

/* L2 norm of a row of D values (D a power of two) in binary32: squares,
 * then pairwise sums (element 2i + element 2i + 1, level by level), then a
 * correctly rounded square root. */
float orc_row_norm_f32(const float* x, int D) {
  float* t = (float*)malloc(sizeof(float) * (size_t)D);
  for (int c = 0; c < D; ++c) t[c] = x[c] * x[c];
  for (int w = D; w > 1; w /= 2)
    for (int i = 0; i < w / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  float r = sqrtf(t[0]);
  free(t);
  return r;
}

/* ------------------------------------------------------------------------ */
/* Window bookkeeping.                                                       */
/* ------------------------------------------------------------------------ */

/* Number of quantized tokens among n: whole groups of G, aligned to token 0,
 * leaving at least R of the most recent tokens in the fp16 window. */
int64_t orc_num_quantized(int64_t n, int G, int R) {
  int64_t over = n - R;
  if (over <= 0) return 0;
  return (over / G) * G;
}

/* With an attention-sink window of S0 tokens: tokens [0, min(n, S0)) stay in
 * fp16, groups of G are aligned to token S0, and at least R of the most
 * recent tokens after the sink stay in fp16. */
int64_t orc_num_quantized_sink(int64_t n, int G, int R, int S0) {
  return n > S0 ? orc_num_quantized(n - S0, G, R) : 0;
}

/* Position-adaptive bit widths of the groups of a slice built by appends of
 * calls[0], calls[1], ... tokens: group g (tokens S0 + gG .. S0 + gG + G - 1,
 * 1-based positions p0 + 1 .. p1 with p1 = S0 + gG + G) is quantized by the
 * first append after which it is quantized, with n = the length after that
 * append; it is recent if p1 > n - delta, else early if p1 <= delta, else
 * middle.  Writes the (key, value) bits of its region for each of the
 * groups quantized after all calls; returns that count or -1. */
int64_t orc_adaptive_group_bits(int G, int R, int S0, int delta, int ncalls, const int64_t* calls,
                                int kb_low, int vb_low, int kb_mid, int vb_mid, int kb_high, int vb_high,
                                uint8_t* group_kbits, uint8_t* group_vbits) {
  if (G <= 0 || R < 0 || S0 < 0 || delta < 0 || ncalls < 0) return -1;
  int64_t n = 0, done = 0;
  for (int c = 0; c < ncalls; ++c) {
    if (calls[c] < 0) return -1;
    n += calls[c];
    int64_t ng = orc_num_quantized_sink(n, G, R, S0) / G;
    for (int64_t g = done; g < ng; ++g) {
      int64_t p1 = (int64_t)S0 + g * G + G;
      int region = p1 > n - delta ? 2 : (p1 <= delta ? 0 : 1);
      group_kbits[g] = (uint8_t)(region == 2 ? kb_high : region == 0 ? kb_low : kb_mid);
      group_vbits[g] = (uint8_t)(region == 2 ? vb_high : region == 0 ? vb_low : vb_mid);
    }
    done = ng;
  }
  return done;
}

/* ------------------------------------------------------------------------ */
/* Drift detection: code histograms and their KL divergence from a          */
/* calibration histogram ("Asymmetric Key-Value Quantization ...", 3.3).     */
/* ------------------------------------------------------------------------ */

/* Adds the histogram of `count` codes (each in [0, 2^bits)) to hist[2^bits].
 * Returns -1 if a code is out of range. */
int orc_code_histogram(const uint16_t* codes, int64_t count, int bits, int64_t* hist) {
  const int nb = 1 << bits;
  for (int64_t i = 0; i < count; ++i) {
    if (codes[i] >= nb) return -1;
    hist[codes[i]] += 1;
  }
  return 0;
}

/* D_KL(p || q) = sum_i p_i ln(p_i / q_i) over nb bins, summed in bin order;
 * bins with p_i = 0 contribute 0, a bin with p_i > 0 and q_i = 0 makes it
 * +inf. */
double orc_kl_divergence(const double* p, const double* q, int nb) {
  double kl = 0.0;
  for (int i = 0; i < nb; ++i) {
    if (p[i] == 0.0) continue;
    if (q[i] == 0.0) return INFINITY;
    kl += p[i] * log(p[i] / q[i]);
  }
  return kl;
}

/* Drift check of ng quantized groups of one slice, canonical codes
 * k_codes / v_codes [ng * G][D].  The calibration histograms are counts
 * (cal_k[2^kbits], cal_v[2^vbits]), turned into probabilities by dividing by
 * their totals; a group's probabilities are its counts divided by G * D.
 * A calibration with no counts at all has no mass in any bin (every q_i = 0,
 * no division), so by the KL rule above every group's KL against it is +inf
 * (a group always has G * D > 0 codes) and its flag is set.
 * Writes kl_k[g], kl_v[g] and flags[g] = (kl_k > thr) | (kl_v > thr) << 1.
 * Returns 0, or -1 on bad arguments (a negative count among them). */
int orc_drift_check(const uint16_t* k_codes, const uint16_t* v_codes, int64_t ng, int G, int D, int kbits,
                    int vbits, const int64_t* cal_k, const int64_t* cal_v, double thr, double* kl_k,
                    double* kl_v, uint8_t* flags) {
  if (ng < 0 || G <= 0 || D <= 0 || kbits < 1 || kbits > 8 || vbits < 1 || vbits > 8) return -1;
  const int nbk = 1 << kbits, nbv = 1 << vbits;
  double qk[256], qv[256], pk[256], pv[256];
  int64_t tk = 0, tv = 0;
  for (int i = 0; i < nbk; ++i) {
    if (cal_k[i] < 0) return -1;
    tk += cal_k[i];
  }
  for (int i = 0; i < nbv; ++i) {
    if (cal_v[i] < 0) return -1;
    tv += cal_v[i];
  }
  for (int i = 0; i < nbk; ++i) qk[i] = tk > 0 ? (double)cal_k[i] / (double)tk : 0.0;
  for (int i = 0; i < nbv; ++i) qv[i] = tv > 0 ? (double)cal_v[i] / (double)tv : 0.0;
  const int64_t per = (int64_t)G * D;
  for (int64_t g = 0; g < ng; ++g) {
    int64_t hk[256] = {0}, hv[256] = {0};
    if (orc_code_histogram(k_codes + g * per, per, kbits, hk) < 0) return -1;
    if (orc_code_histogram(v_codes + g * per, per, vbits, hv) < 0) return -1;
    for (int i = 0; i < nbk; ++i) pk[i] = (double)hk[i] / (double)per;
    for (int i = 0; i < nbv; ++i) pv[i] = (double)hv[i] / (double)per;
    kl_k[g] = orc_kl_divergence(pk, qk, nbk);
    kl_v[g] = orc_kl_divergence(pv, qv, nbv);
    flags[g] = (uint8_t)((kl_k[g] > thr ? 1 : 0) | (kl_v[g] > thr ? 2 : 0));
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Encode one (batch, kv-head) slice of n tokens into canonical arrays.      */
/* ------------------------------------------------------------------------ */

/* k, v: [n][D] elements of `dtype` (0 f32, 1 f16, 2 bf16).
 * Canonical outputs (nq = orc_num_quantized(n, G, R), nr = n - nq):
 *   k_codes [nq][D] (one code per uint16)   k_scale, k_zero [nq/G][D] fp16 bits
 *   v_codes [nq][D]                         v_scale, v_zero [nq][D/G] fp16 bits
 *   k_resid, v_resid [nr][D] fp16 bits
 * Entry: each element is widened to binary32; keys are rotated first when
 * `rotate` is set; then every element is rounded to fp16 and only the fp16
 * values are seen downstream.  Returns nq, or -1 on bad arguments. */
int64_t orc_encode_slice(const void* k, const void* v, int dtype, int64_t n, int D,
                         int kbits, int vbits, int G, int R, int rotate,
                         uint16_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                         uint16_t* v_codes, uint16_t* v_scale, uint16_t* v_zero,
                         uint16_t* k_resid, uint16_t* v_resid) {
  return orc_encode_slice_ext(k, v, dtype, n, D, kbits, vbits, G, R, rotate, 0, 0, 0, k_codes, k_scale,
                              k_zero, v_codes, v_scale, v_zero, k_resid, v_resid, NULL, NULL, NULL, NULL, NULL);
}

/* As orc_encode_slice, with an attention-sink window of S0 tokens (0: none)
 * and, if `hybrid`, the per-group symmetric/asymmetric choice.  The
 * quantized tokens are [s, s + nq) with s = min(n, S0) and
 * nq = orc_num_quantized_sink(n, G, R, S0); k_resid / v_resid hold the other
 * n - nq tokens in position order (the sink, then the recent window).
 * k_sym [nq/G][D] and v_sym [nq][D/G] (may be NULL) receive 1 where a group
 * took the symmetric quantizer.  With `token_norm`, each quantized key token
 * is divided by its norm (orc_row_norm_f32 of its fp16 row) and rounded to
 * fp16 before the key quantizer, and k_norm [nq] receives the norms as fp16
 * bits (0 for a zero row, whose normalized values are 0).  group_kbits /
 * group_vbits [nq/G] (may be NULL) give per-group bit widths in place of
 * kbits / vbits (position-adaptive caches, see orc_adaptive_group_bits). */
int64_t orc_encode_slice_ext(const void* k, const void* v, int dtype, int64_t n, int D,
                             int kbits, int vbits, int G, int R, int rotate, int S0, int hybrid,
                             int token_norm, uint16_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                             uint16_t* v_codes, uint16_t* v_scale, uint16_t* v_zero,
                             uint16_t* k_resid, uint16_t* v_resid, uint8_t* k_sym, uint8_t* v_sym,
                             uint16_t* k_norm, const uint8_t* group_kbits, const uint8_t* group_vbits) {
  if (n < 0 || D <= 0 || G <= 0 || R < 0 || D % G != 0 || S0 < 0) return -1;
  if (kbits < 1 || kbits > 16 || vbits < 1 || vbits > 16) return -1;
  if (hybrid && (kbits < 2 || vbits < 2)) return -1;
  if ((rotate || token_norm) && (D & (D - 1)) != 0) return -1;
  if (token_norm && !k_norm) return -1;
  int64_t nq = orc_num_quantized_sink(n, G, R, S0);
  int64_t s0 = n < S0 ? n : S0;
  float* kt = (float*)malloc(sizeof(float) * (size_t)n * (size_t)D + 1);
  float* vt = (float*)malloc(sizeof(float) * (size_t)n * (size_t)D + 1);
  float* row = (float*)malloc(sizeof(float) * (size_t)D);
  float* grp = (float*)malloc(sizeof(float) * (size_t)(G > D ? G : D));
  uint16_t* cod = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(G > D ? G : D));
  if (!kt || !vt || !row || !grp || !cod) { free(kt); free(vt); free(row); free(grp); free(cod); return -1; }

  /* entry conversion */
  for (int64_t t = 0; t < n; ++t) {
    for (int c = 0; c < D; ++c) row[c] = load_in(k, dtype, (size_t)t * D + c);
    if (rotate) orc_fwht_f32(row, D);
    for (int c = 0; c < D; ++c) kt[t * D + c] = orc_f16_to_f32(orc_f32_to_f16(row[c]));
    for (int c = 0; c < D; ++c)
      vt[t * D + c] = orc_f16_to_f32(orc_f32_to_f16(load_in(v, dtype, (size_t)t * D + c)));
  }

  /* token-norm scaling of the quantized keys (the fp16 window keeps them as
   * they are) */
  float* kq = (float*)malloc(sizeof(float) * (size_t)(nq > 0 ? nq : 1) * (size_t)D);
  for (int64_t t = 0; t < nq; ++t) {
    const float* x = kt + (s0 + t) * D;
    float* y = kq + t * D;
    if (!token_norm) {
      for (int c = 0; c < D; ++c) y[c] = x[c];
      continue;
    }
    float nrm = orc_row_norm_f32(x, D);
    k_norm[t] = orc_f32_to_f16(nrm);
    for (int c = 0; c < D; ++c) y[c] = nrm == 0.0f ? 0.0f : orc_f16_to_f32(orc_f32_to_f16(x[c] / nrm));
  }

  /* keys: per channel, groups of G consecutive tokens (token s0 + q for
   * quantized index q) */
  for (int64_t g = 0; g < nq / G; ++g)
    for (int c = 0; c < D; ++c) {
      const int kb = group_kbits ? group_kbits[g] : kbits;
      for (int i = 0; i < G; ++i) grp[i] = kq[(g * G + i) * D + c];
      int sym = 0;
      if (hybrid)
        sym = orc_quantize_group_hybrid(grp, G, kb, cod, &k_scale[g * D + c], &k_zero[g * D + c]);
      else
        orc_quantize_group(grp, G, kb, cod, NULL, NULL, &k_scale[g * D + c], &k_zero[g * D + c]);
      if (k_sym) k_sym[g * D + c] = (uint8_t)sym;
      for (int i = 0; i < G; ++i) k_codes[(g * G + i) * D + c] = cod[i];
    }

  /* values: per token, groups of G consecutive channels */
  int ng = D / G;
  for (int64_t t = 0; t < nq; ++t)
    for (int j = 0; j < ng; ++j) {
      const int vb = group_vbits ? group_vbits[t / G] : vbits;
      for (int i = 0; i < G; ++i) grp[i] = vt[(s0 + t) * D + j * G + i];
      int sym = 0;
      if (hybrid)
        sym = orc_quantize_group_hybrid(grp, G, vb, cod, &v_scale[t * ng + j], &v_zero[t * ng + j]);
      else
        orc_quantize_group(grp, G, vb, cod, NULL, NULL, &v_scale[t * ng + j], &v_zero[t * ng + j]);
      if (v_sym) v_sym[t * ng + j] = (uint8_t)sym;
      for (int i = 0; i < G; ++i) v_codes[t * D + j * G + i] = cod[i];
    }

  /* fp16 tokens in position order: the sink [0, s0), then the window */
  int64_t r = 0;
  for (int64_t t = 0; t < n; ++t) {
    if (t >= s0 && t < s0 + nq) continue;
    for (int c = 0; c < D; ++c) {
      k_resid[r * D + c] = orc_f32_to_f16(kt[t * D + c]);
      v_resid[r * D + c] = orc_f32_to_f16(vt[t * D + c]);
    }
    ++r;
  }

  free(kq);
  free(kt); free(vt); free(row); free(grp); free(cod);
  return nq;
}

/* ------------------------------------------------------------------------ */
/* Canonical code packing.                                                   */
/* ------------------------------------------------------------------------ */

/* Codes of one token row are packed along channels into a little-endian
 * bit stream: the code of channel c occupies stream bits [b*c, b*c + b),
 * stream bit i being bit (i mod 8) of byte floor(i / 8).  Row bytes =
 * ceil(D*b/8).  For b dividing 8 this puts channel c at bit b*(c mod 8/b)
 * of byte floor(b*c/8). */
void orc_pack_codes(const uint16_t* codes, int64_t rows, int D, int bits, uint8_t* out) {
  int64_t rb = ((int64_t)D * bits + 7) / 8;
  memset(out, 0, (size_t)(rows * rb));
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < D; ++c)
      for (int i = 0; i < bits; ++i)
        if ((codes[r * D + c] >> i) & 1u) {
          int64_t bit = (int64_t)c * bits + i;
          out[r * rb + bit / 8] |= (uint8_t)(1u << (bit % 8));
        }
}

void orc_unpack_codes(const uint8_t* in, int64_t rows, int D, int bits, uint16_t* codes) {
  int64_t rb = ((int64_t)D * bits + 7) / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < D; ++c) {
      uint16_t v = 0;
      for (int i = 0; i < bits; ++i) {
        int64_t bit = (int64_t)c * bits + i;
        if ((in[r * rb + bit / 8] >> (bit % 8)) & 1u) v |= (uint16_t)(1u << i);
      }
      codes[r * D + c] = v;
    }
}

/* ------------------------------------------------------------------------ */
/* Decode and attention in fp64 ("Asymmetric Key-Value Quantization ...",    */
/* section 1: softmax(q K^T / sqrt(d)) V).                                   */
/* ------------------------------------------------------------------------ */

/* Dequantized key / value element of token t, channel c (fp64). */
static double key_at(int64_t t, int c, int64_t nq, int D, int G,
                     const uint16_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                     const uint16_t* k_resid, const uint16_t* k_norm) {
  if (t < nq) {
    int64_t g = t / G;
    double k = (double)orc_f16_to_f32(k_zero[g * D + c]) +
               (double)k_codes[t * D + c] * (double)orc_f16_to_f32(k_scale[g * D + c]);
    return k_norm ? k * (double)orc_f16_to_f32(k_norm[t]) : k;
  }
  return (double)orc_f16_to_f32(k_resid[(t - nq) * D + c]);
}

static double value_at(int64_t t, int c, int64_t nq, int D, int G,
                       const uint16_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                       const uint16_t* v_resid) {
  if (t < nq) {
    int ng = D / G;
    int j = c / G;
    return (double)orc_f16_to_f32(v_zero[t * ng + j]) +
           (double)v_codes[t * D + c] * (double)orc_f16_to_f32(v_scale[t * ng + j]);
  }
  return (double)orc_f16_to_f32(v_resid[(t - nq) * D + c]);
}

/* Unnormalized attention statistics over tokens [t0, t1) of the canonical
 * order (the nq quantized tokens, then the n - nq fp16 tokens) for nh query
 * heads q[nh][D] (fp64, already rotated if the keys were):
 *   sigma_t = (sum_c q_c khat_tc) / sqrt(D)
 *   m = max sigma_t (-inf on an empty range), w_t = exp(sigma_t - m)
 *   l = sum w_t, o_c = sum w_t vhat_tc            (sums in token order)
 * m[nh], l[nh], o[nh][D]. */
void orc_attend_partial(const double* q, int nh, int64_t n, int64_t nq, int D, int G,
                        const uint16_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                        const uint16_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                        const uint16_t* k_resid, const uint16_t* v_resid, const uint16_t* k_norm,
                        int64_t t0, int64_t t1, double* m, double* l, double* o) {
  (void)n;
  double inv_sqrt_d = 1.0 / sqrt((double)D);
  int64_t cnt = t1 > t0 ? t1 - t0 : 0;
  double* sig = (double*)malloc(sizeof(double) * (size_t)(cnt + 1));
  for (int h = 0; h < nh; ++h) {
    const double* qh = q + (size_t)h * D;
    double mx = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
      double s = 0.0;
      for (int c = 0; c < D; ++c)
        s += qh[c] * key_at(t, c, nq, D, G, k_codes, k_scale, k_zero, k_resid, k_norm);
      s *= inv_sqrt_d;
      sig[t - t0] = s;
      if (s > mx) mx = s;
    }
    double L = 0.0;
    double* oh = o + (size_t)h * D;
    for (int c = 0; c < D; ++c) oh[c] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      double w = exp(sig[t - t0] - mx);
      L += w;
      for (int c = 0; c < D; ++c)
        oh[c] += w * value_at(t, c, nq, D, G, v_codes, v_scale, v_zero, v_resid);
    }
    m[h] = mx;
    l[h] = L;
  }
  free(sig);
}

/* Full attention over all n tokens: out[nh][D] = o / l. */
void orc_attend_slice(const double* q, int nh, int64_t n, int64_t nq, int D, int G,
                      const uint16_t* k_codes, const uint16_t* k_scale, const uint16_t* k_zero,
                      const uint16_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                      const uint16_t* k_resid, const uint16_t* v_resid, const uint16_t* k_norm,
                      double* out) {
  double* m = (double*)malloc(sizeof(double) * (size_t)nh);
  double* l = (double*)malloc(sizeof(double) * (size_t)nh);
  orc_attend_partial(q, nh, n, nq, D, G, k_codes, k_scale, k_zero, v_codes, v_scale, v_zero,
                     k_resid, v_resid, k_norm, 0, n, m, l, out);
  for (int h = 0; h < nh; ++h)
    for (int c = 0; c < D; ++c) out[(size_t)h * D + c] /= l[h];
  free(m);
  free(l);
}

/* Merge S partial results (m[s][nh], l[s][nh], o[s][nh][D]) of disjoint token
 * ranges: M = max_s m_s, out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
 * A split with m = -inf (empty) contributes nothing. */
void orc_merge_partials(int S, int nh, int D, const double* m, const double* l, const double* o,
                        double* out) {
  for (int h = 0; h < nh; ++h) {
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (m[s * nh + h] > M) M = m[s * nh + h];
    double L = 0.0;
    for (int c = 0; c < D; ++c) out[(size_t)h * D + c] = 0.0;
    for (int s = 0; s < S; ++s) {
      double ms = m[s * nh + h];
      if (ms == -INFINITY) continue;
      double a = exp(ms - M);
      L += a * l[s * nh + h];
      for (int c = 0; c < D; ++c) out[(size_t)h * D + c] += a * o[((size_t)s * nh + h) * D + c];
    }
    for (int c = 0; c < D; ++c) out[(size_t)h * D + c] /= L;
  }
}

/* ------------------------------------------------------------------------ */
/* Bits per element ("Asymmetric Key-Value Quantization ...", sections 3.1,  */
/* 3.4), counting `overhead_bits` of parameters per group of G elements and  */
/* 16 bits per element of the fp16 window, over both K and V:                */
/*   bpe = [nq (bk + ovh/G) + nq (bv + ovh/G) + 2*16*nr] / (2n)              */
/* ------------------------------------------------------------------------ */
double orc_bits_per_element(int64_t n, int kbits, int vbits, int G, int R, double overhead_bits) {
  return orc_bits_per_element_sink(n, kbits, vbits, G, R, 0, overhead_bits);
}

/* The same with an fp16 attention-sink window of S0 tokens. */
double orc_bits_per_element_sink(int64_t n, int kbits, int vbits, int G, int R, int S0,
                                 double overhead_bits) {
  if (n <= 0) return 0.0;
  int64_t nq = orc_num_quantized_sink(n, G, R, S0);
  int64_t nr = n - nq;
  double q = (double)nq * (kbits + overhead_bits / G) + (double)nq * (vbits + overhead_bits / G);
  return (q + 2.0 * 16.0 * (double)nr) / (2.0 * (double)n);
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the Python wrapper.                                     */
/* ------------------------------------------------------------------------ */
void orc_f32_to_f16_n(const float* x, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = orc_f32_to_f16(x[i]);
}
void orc_f16_to_f32_n(const uint16_t* h, float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = orc_f16_to_f32(h[i]);
}
void orc_bf16_to_f32_n(const uint16_t* b, float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = orc_bf16_to_f32(b[i]);
}
void orc_f32_to_bf16_n(const float* x, uint16_t* b, int64_t n) {
  for (int64_t i = 0; i < n; ++i) b[i] = orc_f32_to_bf16(x[i]);
}
