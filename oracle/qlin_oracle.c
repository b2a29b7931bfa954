/*
 * qlin CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of what the quantized
 * linear layer computes. It exists so that tests, the smoke check and the
 * benchmark's CPU-baseline leg can check and time the GPU library against it.
 * The product path (the HIP library and its Python binding) never loads,
 * links or calls this file, and this file includes nothing from the product.
 *
 * Sources (web pages on the weight-format linear layer; cited by page title
 * and section):
 *   [E2B]  "MI300X ... Gemma 4 E2B: fp8 fastest, yet farthest from the
 *          original weights" (geoz.com.cn article), sections "Ten builds",
 *          "Step 1: build the formats", "Step 2: the card's matmuls",
 *          "How close are they to the trained weights?",
 *          "Tip: E4M3 or E4M3FNUZ".
 *   [SIZES] "Gemma 4 From E2B to 31B on an AMD MI300X" (dev.to), sections
 *          "The Sizes and the Builds" (format table), "Step 1 -- Build the
 *          Larger Repacks" (expert bank split), "The 4-Bit Builds Stay Slow".
 *   [CARD] "Gemma 4 31B-it QAT, FP8 E4M3 W8A8, text only" model card,
 *          intro paragraph and the "Measured against the QAT weights" table.
 *   [PR]   vLLM PR #45854 report ("Enable fp8_per_channel ... on mi300x"),
 *          per-token activation / per-output-channel weight quant config.
 *
 * Precision: fp32 with k-ascending accumulation for the floating-point
 * GEMMs, int32 for the int8 GEMM, IEEE fp32 division in every quantizer,
 * E4M3 round-to-nearest-even with saturation; statistics in fp64.
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math).
 *
 * Readings taken where the pages are silent:
 *   - int4 codes are signed [-8,7], stored offset-binary u = c + 8, two per
 *     byte, low nibble = even k; one bf16 step per (row, 32 values).
 *   - q4_0 step recovery keeps the smallest step that reproduces every
 *     stored bf16 value of the group.
 *   - scales are absmax/FMAX with no headroom (FMAX 448 OCP, 240 FNUZ,
 *     127 int8); an all-zero row has scale 0 and codes 0.
 *   - negative values that round to zero give 0x80 in OCP E4M3 and 0x00
 *     in E4M3FNUZ (which has no negative zero).
 *   - epilogues are (float(acc) * s_a) * s_w, two fp32 roundings, then
 *     bf16 round-to-nearest-even.
 *   - W4A16 dequantises each weight to bf16(c * step) before the multiply.
 *   - MoE: gate rows then up rows in the fused gate_up bank; SiLU(g)*u in
 *     fp32, requantised per (token, expert) from fp32; down; combine in
 *     slot order with the router probabilities, not renormalised.
 *   - online per-channel quantisation of bf16 weights is the per-token
 *     activation quantiser applied to each output channel (row of W).
 *   - SwiGLU-OAI (alpha, beta, clamp limit named by [PR], formula not on the
 *     page) is the published form: gate clamped from above at the limit, up
 *     clamped to [-limit, limit], act = gate * sigmoid(alpha * gate) *
 *     (up + beta).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QO_OCP 0
#define QO_FNUZ 1
#define QO_INT8 2

#define QO_ACT_SILU 0
#define QO_ACT_SWIGLU_OAI 1

/* ------------------------------------------------------------------------ */
/* bf16                                                                     */
/* ------------------------------------------------------------------------ */

static float bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Nearest bf16 to a finite float, ties to the even bf16 pattern. Written as
 * an explicit choice between the two bf16 neighbours of x. */
static uint16_t bf16_nearest(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint16_t lo = (uint16_t)(u >> 16); /* truncated: neighbour toward zero */
  if ((u & 0xFFFFu) == 0) return lo;
  uint16_t hi = (uint16_t)(lo + 1); /* neighbour away from zero */
  double dlo = fabs((double)x - (double)bf16_value(lo));
  double dhi = fabs((double)bf16_value(hi) - (double)x);
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1) ? hi : lo;
}

float qo_bf16_value(uint16_t b) { return bf16_value(b); }
uint16_t qo_bf16_nearest(float x) { return bf16_nearest(x); }

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP) and E4M3FNUZ  -- [E2B] "Tip: E4M3 or E4M3FNUZ": same three */
/* mantissa bits, FNUZ tops out at 240 instead of 448 and has no -0.       */
/* ------------------------------------------------------------------------ */

/* Decode a code from its bit fields s eeee mmm. */
double qo_fp8_value(uint8_t b, int fmt) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (fmt == QO_FNUZ) {
    if (b == 0x80) return NAN; /* the single NaN, no negative zero */
    v = (e == 0) ? ldexp((double)m, -10) : ldexp(1.0 + m / 8.0, e - 8);
  } else {
    if (e == 15 && m == 7) return NAN; /* 0x7F / 0xFF */
    v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  }
  return s ? -v : v;
}

/* fp32 value of a code (exact: at most 4 significant bits). */
static float fp8_f(uint8_t b, int fmt) { return (float)qo_fp8_value(b, fmt); }

/* Nearest representable magnitude, ties to the even code (even mantissa
 * LSB), saturating at the largest finite code. Codes 0..top increase
 * monotonically in value, so a bisection over the decoded table finds the
 * two neighbours. */
uint8_t qo_fp8_encode(float x, int fmt) {
  const int top = (fmt == QO_FNUZ) ? 0x7F : 0x7E;
  double a = fabs((double)x);
  int neg = signbit(x) ? 1 : 0;
  int mag;
  if (a >= qo_fp8_value((uint8_t)top, fmt)) {
    mag = top;
  } else {
    int lo = 0, hi = top; /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
      int mid = (lo + hi) / 2;
      if (qo_fp8_value((uint8_t)mid, fmt) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - qo_fp8_value((uint8_t)lo, fmt);
    double dhi = qo_fp8_value((uint8_t)hi, fmt) - a;
    if (dlo < dhi) mag = lo;
    else if (dhi < dlo) mag = hi;
    else mag = (lo % 2 == 0) ? lo : hi;
  }
  if (mag == 0) return (uint8_t)((neg && fmt == QO_OCP) ? 0x80 : 0x00);
  return (uint8_t)(mag | (neg << 7));
}

void qo_fp8_encode_array(const float* x, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = qo_fp8_encode(x[i], fmt);
}

void qo_bf16_nearest_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_nearest(x[i]);
}

/* ------------------------------------------------------------------------ */
/* int8: symmetric, 255 levels per row ([E2B] fidelity section), RNE.       */
/* ------------------------------------------------------------------------ */
static int8_t int8_code(float v) {
  float r = rintf(v); /* default rounding mode: nearest even */
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

/* ------------------------------------------------------------------------ */
/* q4_0 repack: recover each group's trained step and its int4 codes without */
/* re-rounding ([E2B] "Step 1"; [SIZES] format table, "int4 holding the QAT */
/* grid exactly").                                                           */
/* ------------------------------------------------------------------------ */

static int nib(const uint8_t* row, int64_t k) {
  uint8_t b = row[k >> 1];
  int u = (k & 1) ? (b >> 4) : (b & 15);
  return u - 8;
}

/* Does `step` reproduce every stored value of the group? Fills codes. */
static int step_reproduces(const uint16_t* w, float step, int8_t* c) {
  if (!(step > 0.0f)) return 0;
  for (int j = 0; j < 32; ++j) {
    float v = bf16_value(w[j]);
    float q = rintf(v / step);
    if (q < -8.0f || q > 7.0f) return 0;
    if (bf16_nearest(q * step) != w[j]) return 0;
    c[j] = (int8_t)q;
  }
  return 1;
}

/* Number of stored values that the nearest codes on `step`, clamped to
 * [-8, 7], reproduce (0 for a step that is not finite and positive). */
static int step_count(const uint16_t* w, float step) {
  if (!(step > 0.0f) || !isfinite(step)) return 0;
  int n = 0;
  for (int j = 0; j < 32; ++j) {
    float q = rintf(bf16_value(w[j]) / step);
    if (q < -8.0f) q = -8.0f;
    if (q > 7.0f) q = 7.0f;
    n += bf16_nearest(q * step) == w[j];
  }
  return n;
}

/* Returns 1 if the group was recovered unambiguously, 0 if it is counted.
 * Writes codes (32) and the bf16 step. */
static int recover_group(const uint16_t* w, int8_t* codes, uint16_t* step_out) {
  float amax = 0.0f;
  for (int j = 0; j < 32; ++j) {
    float a = fabsf(bf16_value(w[j]));
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    memset(codes, 0, 32);
    *step_out = 0;
    return 0;
  }
  /* A value whose code is +-1, +-2, +-4 or -8 equals step * 2^p exactly, so
   * the step is among |w_i| / p for p in {1,2,4,8}. */
  float best = INFINITY, second = INFINITY;
  int8_t tmp[32];
  static const float P[4] = {1.0f, 2.0f, 4.0f, 8.0f};
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(bf16_value(w[i]));
    if (a == 0.0f) continue;
    for (int p = 0; p < 4; ++p) {
      float s = a / P[p];
      if (s == best || s == second) continue;
      if (step_reproduces(w, s, tmp)) {
        if (s < best) { second = best; best = s; }
        else if (s < second) second = s;
      }
    }
  }
  int exact = isfinite(best) && !isfinite(second);
  if (!isfinite(best)) {
    /* No power-of-two code in the group: search around |w|max / |c|max for
     * the remaining code magnitudes. */
    static const float A[4] = {3.0f, 5.0f, 6.0f, 7.0f};
    for (int ai = 0; ai < 4; ++ai) {
      uint16_t c0 = bf16_nearest(amax / A[ai]);
      for (int d = -8; d <= 8; ++d) {
        float s = bf16_value((uint16_t)(c0 + d));
        if (step_reproduces(w, s, tmp) && s < best) best = s;
      }
    }
  }
  if (!isfinite(best)) {
    /* No bf16 step puts the whole group on a 4-bit grid (a trained step that
     * is not a bf16 value does this: bf16(c * step) rounds c * step for some
     * codes). Keep the candidate step -- |w_i| / p and the neighbours above --
     * whose nearest codes reproduce the most stored values, the smaller step
     * on ties; codes are nearest on it, clamped to [-8, 7]. */
    int most = -1;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(bf16_value(w[i]));
      if (a == 0.0f) continue;
      for (int p = 0; p < 4; ++p) {
        float s = a / P[p];
        int n = step_count(w, s);
        if (n > most || (n == most && s < best)) { most = n; best = s; }
      }
    }
    static const float A[4] = {3.0f, 5.0f, 6.0f, 7.0f};
    for (int ai = 0; ai < 4; ++ai) {
      uint16_t c0 = bf16_nearest(amax / A[ai]);
      for (int d = -8; d <= 8; ++d) {
        float s = bf16_value((uint16_t)(c0 + d));
        if (!(s > 0.0f) || !isfinite(s)) continue;
        int n = step_count(w, s);
        if (n > most || (n == most && s < best)) { most = n; best = s; }
      }
    }
    for (int j = 0; j < 32; ++j) {
      float q = rintf(bf16_value(w[j]) / best);
      if (q < -8.0f) q = -8.0f;
      if (q > 7.0f) q = 7.0f;
      codes[j] = (int8_t)q;
    }
    *step_out = bf16_nearest(best);
    return 0;
  }
  step_reproduces(w, best, codes);
  *step_out = bf16_nearest(best); /* best is a bf16 value already */
  return exact;
}

void qo_repack_q4_0(const uint16_t* w, int64_t N, int64_t K, uint8_t* packed,
                    uint16_t* steps, int64_t* n_ambiguous) {
  int64_t G = K / 32, amb = 0;
#pragma omp parallel for reduction(+ : amb) schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int8_t c[32];
    for (int64_t g = 0; g < G; ++g) {
      if (!recover_group(w + n * K + g * 32, c, &steps[n * G + g])) amb++;
      for (int j = 0; j < 32; j += 2) {
        uint8_t lo = (uint8_t)(c[j] + 8), hi = (uint8_t)(c[j + 1] + 8);
        packed[n * (K / 2) + g * 16 + j / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
  if (n_ambiguous) *n_ambiguous = amb;
}

void qo_unpack_q4(const uint8_t* packed, int64_t N, int64_t K, int8_t* codes) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) codes[n * K + k] = (int8_t)nib(packed + n * (K / 2), k);
}

/* Grid value c * step in fp32 (exact: <= 4 + 8 significant bits). */
static float grid_value(const uint8_t* prow, const uint16_t* srow, int64_t k) {
  return (float)nib(prow, k) * bf16_value(srow[k / 32]);
}

/* ------------------------------------------------------------------------ */
/* FP8 per-channel repack ([E2B] "Step 1", verify report; [CARD] intro:     */
/* E4M3, one float32 scale per output channel, no calibration data).        */
/* s_w = absmax / FMAX, q = enc(w / s_w).                                    */
/* ------------------------------------------------------------------------ */
void qo_repack_fp8(const uint8_t* packed, const uint16_t* steps, int64_t N, int64_t K, int fmt,
                   uint8_t* wq, float* wscale) {
  const float FMAX = (fmt == QO_FNUZ) ? 240.0f : 448.0f;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* pr = packed + n * (K / 2);
    const uint16_t* sr = steps + n * (K / 32);
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float a = fabsf(grid_value(pr, sr, k));
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      wscale[n] = 0.0f;
      memset(wq + n * K, 0, (size_t)K);
      continue;
    }
    float s = amax / FMAX;
    wscale[n] = s;
    for (int64_t k = 0; k < K; ++k) wq[n * K + k] = qo_fp8_encode(grid_value(pr, sr, k) / s, fmt);
  }
}

/* int8 per-channel repack ([SIZES] format table "int8 weights per channel";
 * [E2B]: 255 levels per row). s_w = absmax / 127, q = clamp(rint(w/s_w)). */
void qo_repack_int8(const uint8_t* packed, const uint16_t* steps, int64_t N, int64_t K,
                    int8_t* wq, float* wscale) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* pr = packed + n * (K / 2);
    const uint16_t* sr = steps + n * (K / 32);
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float a = fabsf(grid_value(pr, sr, k));
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      wscale[n] = 0.0f;
      memset(wq + n * K, 0, (size_t)K);
      continue;
    }
    float s = amax / 127.0f;
    wscale[n] = s;
    for (int64_t k = 0; k < K; ++k) wq[n * K + k] = int8_code(grid_value(pr, sr, k) / s);
  }
}

/* Repack fidelity against the QAT grid values c*step ([E2B] verify report
 * fields relative_rms_error and max_rel_err; [CARD] "largest error, as a
 * fraction of its row's largest value"). fmt: QO_OCP/QO_FNUZ (wq are fp8
 * codes) or QO_INT8. Sums in fp64. */
void qo_repack_stats(const uint8_t* packed, const uint16_t* steps, const void* wq,
                     const float* wscale, int64_t N, int64_t K, int fmt, double* rel_rms,
                     double* max_rel) {
  double num = 0.0, den = 0.0, mx = 0.0;
#pragma omp parallel for reduction(+ : num, den) reduction(max : mx) schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* pr = packed + n * (K / 2);
    const uint16_t* sr = steps + n * (K / 32);
    double amax = 0.0, emax = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double w = grid_value(pr, sr, k);
      double d = (fmt == QO_INT8) ? (double)((const int8_t*)wq)[n * K + k]
                                  : qo_fp8_value(((const uint8_t*)wq)[n * K + k], fmt);
      double e = d * (double)wscale[n] - w;
      num += e * e;
      den += w * w;
      if (fabs(w) > amax) amax = fabs(w);
      if (fabs(e) > emax) emax = fabs(e);
    }
    if (amax > 0.0 && emax / amax > mx) mx = emax / amax;
  }
  *rel_rms = den > 0.0 ? sqrt(num / den) : 0.0;
  *max_rel = mx;
}

/* Share of bf16(c * step_stored) equal bit for bit to the stored bf16 QAT
 * values ([E2B] key conclusions: share of values bit-identical). */
double qo_frac_bit_identical(const uint8_t* packed, const uint16_t* steps, const uint16_t* w,
                             int64_t N, int64_t K) {
  int64_t same = 0;
#pragma omp parallel for reduction(+ : same) schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      same += bf16_nearest(grid_value(packed + n * (K / 2), steps + n * (K / 32), k)) == w[n * K + k];
  return (double)same / (double)(N * K);
}

/* ------------------------------------------------------------------------ */
/* E4M3FNUZ -> OCP E4M3 ([E2B] "Tip: E4M3 or E4M3FNUZ": vLLM converts the    */
/* format at load time; here the opposite direction, since this GPU's FP8   */
/* is OCP). Per row, exact when possible, else nearest-even and counted.    */
/* ------------------------------------------------------------------------ */
void qo_fnuz_to_ocp(const uint8_t* win, const float* sin, int64_t N, int64_t K, uint8_t* wout,
                    float* sout, int64_t* n_inexact) {
  int64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* r = win + n * K;
    int has240 = 0;
    for (int64_t k = 0; k < K; ++k)
      if ((r[k] & 0x7F) == 0x7F) has240 = 1;
    if (!has240) {
      /* Same bits decode to exactly twice the value in OCP (bias 7 vs 8,
       * subnormal quantum 2^-9 vs 2^-10): halve the scale. */
      for (int64_t k = 0; k < K; ++k) {
        if (r[k] == 0x80) { bad++; wout[n * K + k] = 0; continue; }
        wout[n * K + k] = r[k];
      }
      sout[n] = sin[n] * 0.5f;
    } else {
      /* Keep the scale and re-encode each value in OCP. */
      for (int64_t k = 0; k < K; ++k) {
        if (r[k] == 0x80) { bad++; wout[n * K + k] = 0; continue; }
        double v = qo_fp8_value(r[k], QO_FNUZ);
        uint8_t o = qo_fp8_encode((float)v, QO_OCP);
        if (v == 0.0) o = 0x00;
        if (qo_fp8_value(o, QO_OCP) != v) bad++;
        wout[n * K + k] = o;
      }
      sout[n] = sin[n];
    }
  }
  if (n_inexact) *n_inexact = bad;
}

/* ------------------------------------------------------------------------ */
/* Dynamic per-token activation quantisation ([CARD] intro: activations     */
/* quantised to FP8 per token at run time; [SIZES] format table: int8       */
/* activations per token). s = absmax / FMAX; q = enc(a / s).               */
/* a: bf16 rows with leading dimension lda. fmt QO_OCP, QO_FNUZ or QO_INT8.  */
/* ------------------------------------------------------------------------ */
static void quant_row_f32(const float* a, int64_t K, int fmt, uint8_t* q, float* s) {
  const float FMAX = fmt == QO_INT8 ? 127.0f : (fmt == QO_FNUZ ? 240.0f : 448.0f);
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k)
    if (fabsf(a[k]) > amax) amax = fabsf(a[k]);
  if (amax == 0.0f) {
    *s = 0.0f;
    memset(q, 0, (size_t)K);
    return;
  }
  float sc = amax / FMAX;
  *s = sc;
  for (int64_t k = 0; k < K; ++k) {
    float v = a[k] / sc;
    q[k] = (fmt == QO_INT8) ? (uint8_t)int8_code(v) : qo_fp8_encode(v, fmt);
  }
}

void qo_quant_act(const uint16_t* a, int64_t M, int64_t K, int64_t lda, int fmt, void* q,
                  float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    float* row = (float*)malloc((size_t)K * sizeof(float));
    for (int64_t k = 0; k < K; ++k) row[k] = bf16_value(a[m * lda + k]);
    quant_row_f32(row, K, fmt, (uint8_t*)q + m * K, &s[m]);
    free(row);
  }
}

/* Online per-channel weight quantisation of bf16 (non-QAT) weights ([PR]:
 * fp8_per_channel enabled for bf16 weights, per_out_ch_quant): one scale per
 * output channel, absmax / FMAX of that row of W [N,K], each weight encoded
 * as w / s. The same quantiser as the per-token activations, on W's rows. */
void qo_quant_weight(const uint16_t* w, int64_t N, int64_t K, int fmt, void* q, float* s) {
  qo_quant_act(w, N, K, K, fmt, q, s);
}

/* Same quantiser on fp32 rows (the MoE intermediate). */
void qo_quant_rows_f32(const float* a, int64_t M, int64_t K, int fmt, void* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) quant_row_f32(a + m * K, K, fmt, (uint8_t*)q + m * K, &s[m]);
}

/* ------------------------------------------------------------------------ */
/* GEMMs. Shapes follow a PyTorch Linear: A [M,K], W [N,K], Y [M,N].         */
/* y32 receives the fp32 result before the final bf16 rounding, y16 the      */
/* bf16 output (either may be NULL).                                         */
/* ------------------------------------------------------------------------ */

/* Row-wise scaled FP8 GEMM ([E2B] "Step 3" kernel RowWiseTorchFP8Scaled-
 * MMLinearKernel; [CARD]: per-channel weight scale, per-token activation
 * scale): y = bf16((sum_k a*w) * s_a[m] * s_w[n]), fp32 accumulation. */
static float tab_ocp[256];
static int tab_ready = 0;
static void tables(void) {
  if (tab_ready) return;
#pragma omp critical(qo_tab)
  {
    if (!tab_ready) {
      for (int b = 0; b < 256; ++b) tab_ocp[b] = fp8_f((uint8_t)b, QO_OCP);
      tab_ready = 1;
    }
  }
}

static float dot_fp8(const uint8_t* a, const uint8_t* w, int64_t K) {
  float acc = 0.0f;
  for (int64_t k = 0; k < K; ++k) acc = acc + tab_ocp[a[k]] * tab_ocp[w[k]];
  return acc;
}

void qo_gemm_fp8(const uint8_t* aq, const float* sa, const uint8_t* wq, const float* sw,
                 int64_t M, int64_t N, int64_t K, float* y32, uint16_t* y16) {
  tables();
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t m = 0; m < M; ++m) {
      float acc = dot_fp8(aq + m * K, wq + n * K, K);
      float y = (acc * sa[m]) * sw[n];
      if (y32) y32[m * N + n] = y;
      if (y16) y16[m * N + n] = bf16_nearest(y);
    }
}

/* int8 W8A8 GEMM ([E2B] "Step 3" kernel TritonInt8ScaledMMLinearKernel;
 * "Step 2": must work for every M, unlike the M > 16 torch path):
 * acc in int32 (exact), y = bf16((float(acc) * s_a) * s_w). */
void qo_gemm_w8a8(const int8_t* aq, const float* sa, const int8_t* wq, const float* sw,
                  int64_t M, int64_t N, int64_t K, int32_t* acc_out, float* y32, uint16_t* y16) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t m = 0; m < M; ++m) {
      int32_t acc = 0;
      for (int64_t k = 0; k < K; ++k) acc += (int32_t)aq[m * K + k] * (int32_t)wq[n * K + k];
      float y = ((float)acc * sa[m]) * sw[n];
      if (acc_out) acc_out[m * N + n] = acc;
      if (y32) y32[m * N + n] = y;
      if (y16) y16[m * N + n] = bf16_nearest(y);
    }
}

/* W4A16 GEMM ([SIZES] "The 4-Bit Builds Stay Slow": the kernel unpacks the
 * weights to bf16 before each multiply; [E2B]: no int4 multiply on the
 * card). wd = bf16(c*step); y = bf16(sum_k a * wd), fp32 accumulation. */
void qo_gemm_w4a16(const uint16_t* a, int64_t lda, const uint8_t* packed, const uint16_t* steps,
                   int64_t M, int64_t N, int64_t K, float* y32, uint16_t* y16) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    float* wd = (float*)malloc((size_t)K * sizeof(float));
    for (int64_t k = 0; k < K; ++k)
      wd[k] = bf16_value(bf16_nearest(grid_value(packed + n * (K / 2), steps + n * (K / 32), k)));
    for (int64_t m = 0; m < M; ++m) {
      float acc = 0.0f;
      for (int64_t k = 0; k < K; ++k) acc = acc + bf16_value(a[m * lda + k]) * wd[k];
      if (y32) y32[m * N + n] = acc;
      if (y16) y16[m * N + n] = bf16_nearest(acc);
    }
    free(wd);
  }
}

/* Plain bf16 GEMM on bf16 weights (the unquantised comparator). */
void qo_gemm_bf16(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t M, int64_t N,
                  int64_t K, float* y32, uint16_t* y16) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t m = 0; m < M; ++m) {
      float acc = 0.0f;
      for (int64_t k = 0; k < K; ++k) acc = acc + bf16_value(a[m * lda + k]) * bf16_value(w[n * K + k]);
      if (y32) y32[m * N + n] = acc;
      if (y16) y16[m * N + n] = bf16_nearest(acc);
    }
}

/* Sampled outputs (for sizes where the full product is too slow): element
 * i is output (mi[i], ni[i]); same arithmetic as the full routines. */
void qo_gemm_fp8_sample(const uint8_t* aq, const float* sa, const uint8_t* wq, const float* sw,
                        int64_t K, const int64_t* mi, const int64_t* ni, int64_t cnt, float* y32) {
  tables();
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < cnt; ++i) {
    float acc = dot_fp8(aq + mi[i] * K, wq + ni[i] * K, K);
    y32[i] = (acc * sa[mi[i]]) * sw[ni[i]];
  }
}

void qo_gemm_w8a8_sample(const int8_t* aq, const float* sa, const int8_t* wq, const float* sw,
                         int64_t K, const int64_t* mi, const int64_t* ni, int64_t cnt,
                         int32_t* acc_out, float* y32) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < cnt; ++i) {
    int32_t acc = 0;
    for (int64_t k = 0; k < K; ++k) acc += (int32_t)aq[mi[i] * K + k] * (int32_t)wq[ni[i] * K + k];
    acc_out[i] = acc;
    y32[i] = ((float)acc * sa[mi[i]]) * sw[ni[i]];
  }
}

void qo_gemm_w4a16_sample(const uint16_t* a, int64_t lda, const uint8_t* packed,
                          const uint16_t* steps, int64_t K, const int64_t* mi, const int64_t* ni,
                          int64_t cnt, float* y32) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < cnt; ++i) {
    float acc = 0.0f;
    const uint8_t* pr = packed + ni[i] * (K / 2);
    const uint16_t* sr = steps + ni[i] * (K / 32);
    for (int64_t k = 0; k < K; ++k)
      acc = acc + bf16_value(a[mi[i] * lda + k]) * bf16_value(bf16_nearest(grid_value(pr, sr, k)));
    y32[i] = acc;
  }
}

/* ------------------------------------------------------------------------ */
/* Mixture-of-experts FP8 block ([SIZES] "Step 1": fused expert banks split  */
/* per expert into gate/up/down, router stays bf16 outside; [PR]: per-token  */
/* activation and per-output-channel weight scales for the fp8 MoE).         */
/* For token t and slot j with expert e = ids[t,j], probability p = probs:   */
/*   h = (x_q . W13_e^T) * s_x[t] * s13[e,:]   (fp32, [2I]: gate then up)     */
/*   act = SiLU(h[:I]) * h[I:]                 (fp32)                         */
/*     or SwiGLU-OAI(h[:I], h[I:]) (the [PR]'s alpha/beta/limit variant)      */
/*   (a_q, s_a) = fp8 per-row quant of act    (from fp32)                    */
/*   d = (a_q . W2_e^T) * s_a * s2[e,:]        (fp32, [H])                    */
/*   y[t] = bf16(sum_j p_j * d_j), slot order j = 0..topk-1.                  */
/* Optional stage outputs (may be NULL): act32 [T*topk, I], aq [T*topk, I],  */
/* sa [T*topk], d32 [T*topk, H], y32 [T, H]; row index t*topk + j.           */
/* ------------------------------------------------------------------------ */
/* SwiGLU-OAI MoE activation ([PR]: gemm1_alpha / gemm1_beta / clamp limit
 * carried into the fused MoE; 1.702 / 1.0 for MiniMax-M3). The gate is
 * clamped from above only, the up value to [-limit, limit]; then
 * gate * sigmoid(alpha * gate), written g / (1 + exp(-alpha g)), times
 * (up + beta). At alpha = 1, beta = 0 and an infinite limit this is the
 * SiLU(g) * u expression below, operation for operation. */
float qo_swiglu_oai(float g, float u, float alpha, float beta, float limit) {
  if (g > limit) g = limit;
  if (u > limit) u = limit;
  if (u < -limit) u = -limit;
  return (g / (1.0f + expf(-(alpha * g)))) * (u + beta);
}

void qo_swiglu_oai_array(const float* g, const float* u, int64_t n, float alpha, float beta,
                         float limit, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = qo_swiglu_oai(g[i], u[i], alpha, beta, limit);
}

static float moe_act(int kind, float g, float u, float alpha, float beta, float limit) {
  if (kind == QO_ACT_SWIGLU_OAI) return qo_swiglu_oai(g, u, alpha, beta, limit);
  const float silu = g / (1.0f + expf(-g));
  return silu * u;
}

static void moe_down_combine(const uint8_t* aq, const float* sa, int64_t T, int64_t H, int64_t I,
                             int topk, const int32_t* ids, const float* probs, const uint8_t* w2,
                             const float* s2, float* d32, float* y32, uint16_t* y16) {
  tables();
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    float* d = (float*)malloc((size_t)(topk * H) * sizeof(float));
    for (int j = 0; j < topk; ++j) {
      int64_t r = t * topk + j, e = ids[r];
      for (int64_t h = 0; h < H; ++h) {
        float acc = dot_fp8(aq + r * I, w2 + (e * H + h) * I, I);
        d[j * H + h] = (acc * sa[r]) * s2[e * H + h];
        if (d32) d32[r * H + h] = d[j * H + h];
      }
    }
    for (int64_t h = 0; h < H; ++h) {
      float y = 0.0f;
      for (int j = 0; j < topk; ++j) y = y + probs[t * topk + j] * d[j * H + h];
      if (y32) y32[t * H + h] = y;
      if (y16) y16[t * H + h] = bf16_nearest(y);
    }
    free(d);
  }
}

/* act = SiLU(g) * u (kind QO_ACT_SILU) or SwiGLU-OAI(g, u) with the given
 * alpha, beta, limit (kind QO_ACT_SWIGLU_OAI), from the dequantised fp32
 * gate and up values. */
void qo_moe_gate_up_act(const uint8_t* xq, const float* sx, int64_t T, int64_t H, int64_t I,
                        int topk, const int32_t* ids, const uint8_t* w13, const float* s13,
                        int kind, float alpha, float beta, float limit, float* act32) {
  tables();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < T * topk; ++r) {
    int64_t t = r / topk, e = ids[r];
    for (int64_t i = 0; i < I; ++i) {
      float g = dot_fp8(xq + t * H, w13 + (e * 2 * I + i) * H, H);
      float u = dot_fp8(xq + t * H, w13 + (e * 2 * I + I + i) * H, H);
      g = (g * sx[t]) * s13[e * 2 * I + i];
      u = (u * sx[t]) * s13[e * 2 * I + I + i];
      act32[r * I + i] = moe_act(kind, g, u, alpha, beta, limit);
    }
  }
}

void qo_moe_gate_up(const uint8_t* xq, const float* sx, int64_t T, int64_t H, int64_t I,
                    int topk, const int32_t* ids, const uint8_t* w13, const float* s13,
                    float* act32) {
  qo_moe_gate_up_act(xq, sx, T, H, I, topk, ids, w13, s13, QO_ACT_SILU, 1.0f, 0.0f, INFINITY, act32);
}

void qo_moe_down(const uint8_t* aq, const float* sa, int64_t T, int64_t H, int64_t I, int topk,
                 const int32_t* ids, const float* probs, const uint8_t* w2, const float* s2,
                 float* d32, float* y32, uint16_t* y16) {
  moe_down_combine(aq, sa, T, H, I, topk, ids, probs, w2, s2, d32, y32, y16);
}

void qo_moe_fp8_act(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                    const int32_t* ids, const float* probs, const uint8_t* w13, const float* s13,
                    const uint8_t* w2, const float* s2, int kind, float alpha, float beta,
                    float limit, float* act32, uint8_t* aq, float* sa, float* d32, float* y32,
                    uint16_t* y16) {
  (void)E;
  int64_t R = T * topk;
  uint8_t* xq = (uint8_t*)malloc((size_t)(T * H));
  float* sx = (float*)malloc((size_t)T * sizeof(float));
  float* act = act32 ? act32 : (float*)malloc((size_t)(R * I) * sizeof(float));
  uint8_t* q = aq ? aq : (uint8_t*)malloc((size_t)(R * I));
  float* s = sa ? sa : (float*)malloc((size_t)R * sizeof(float));
  qo_quant_act(x, T, H, H, QO_OCP, xq, sx);
  qo_moe_gate_up_act(xq, sx, T, H, I, topk, ids, w13, s13, kind, alpha, beta, limit, act);
  qo_quant_rows_f32(act, R, I, QO_OCP, q, s);
  moe_down_combine(q, s, T, H, I, topk, ids, probs, w2, s2, d32, y32, y16);
  if (!act32) free(act);
  if (!aq) free(q);
  if (!sa) free(s);
  free(xq);
  free(sx);
}

void qo_moe_fp8(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                const int32_t* ids, const float* probs, const uint8_t* w13, const float* s13,
                const uint8_t* w2, const float* s2, float* act32, uint8_t* aq, float* sa,
                float* d32, float* y32, uint16_t* y16) {
  qo_moe_fp8_act(x, T, H, I, E, topk, ids, probs, w13, s13, w2, s2, QO_ACT_SILU, 1.0f, 0.0f,
                 INFINITY, act32, aq, sa, d32, y32, y16);
}

/* ------------------------------------------------------------------------ */
/* int4 vocabulary table lookup ([E2B] tip on the int4 vocabulary tables,  */
/* [SIZES] "Tip: int4 Embedding Tables Cost More at Larger Sizes"):         */
/* embed_tokens, the untied lm_head and the per-layer embeddings are        */
/* packed int4 in groups of 32, as trained). out[t] = bf16(c * step) of row  */
/* ids[t] of the table (packed [V][D/2], steps [V][D/32]); a row id outside  */
/* [0, V) gives a row of zeros. The untied lm_head is the W4A16 GEMM above.  */
/* ------------------------------------------------------------------------ */
void qo_embed_q4(const int32_t* ids, int64_t T, const uint8_t* packed, const uint16_t* steps,
                 int64_t V, int64_t D, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const int64_t r = ids[t];
    for (int64_t k = 0; k < D; ++k)
      out[t * D + k] = (r < 0 || r >= V)
                           ? 0
                           : bf16_nearest(grid_value(packed + r * (D / 2), steps + r * (D / 32), k));
  }
}

/* ------------------------------------------------------------------------ */
/* Mixture-of-experts W4A16 block ([SIZES] "The 4-Bit Builds Stay Slow": the */
/* 4-bit MoE runs a WNA16 expert path -- bf16 activations, group-32 int4     */
/* expert weights unpacked to bf16 -- on the fused gate_up / down banks split */
/* per expert as in "Step 1"). The steps of the fp8 block without activation  */
/* quantisation; the down projection takes bf16 activations, so the SiLU*up  */
/* product is rounded to bf16 once. Weights: p13 [E][2I][H/2] packed codes,  */
/* st13 [E][2I][H/32] bf16 steps (rows 0..I-1 gate, I..2I-1 up); p2          */
/* [E][H][I/2], st2 [E][H][I/32]. wd = bf16(c*step) as in the W4A16 GEMM.    */
/* For token t and slot j with expert e = ids[t,j], probability p = probs:   */
/*   h = x . W13d_e^T               (fp32, k ascending; [2I])                */
/*   act = bf16(SiLU(h[:I]) * h[I:])                                         */
/*   d = act . W2d_e^T              (fp32, [H])                              */
/*   y[t] = bf16(sum_j p_j * d_j), slot order j = 0..topk-1.                  */
/* Stage outputs (may be NULL): act16 [T*topk, I] bf16 bits, d32             */
/* [T*topk, H], y32 [T, H]; row index t*topk + j.                            */
/* ------------------------------------------------------------------------ */
void qo_moe_w4a16(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                  const int32_t* ids, const float* probs, const uint8_t* p13, const uint16_t* st13,
                  const uint8_t* p2, const uint16_t* st2, uint16_t* act16, float* d32, float* y32,
                  uint16_t* y16) {
  (void)E;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    float* wrow = (float*)malloc((size_t)(H > I ? H : I) * sizeof(float));
    uint16_t* act = (uint16_t*)malloc((size_t)I * sizeof(uint16_t));
    float* d = (float*)malloc((size_t)(topk * H) * sizeof(float));
    for (int j = 0; j < topk; ++j) {
      const int64_t r = t * topk + j, e = ids[r];
      for (int64_t i = 0; i < I; ++i) {
        float g = 0.0f, u = 0.0f;
        const int64_t rg = e * 2 * I + i, ru = e * 2 * I + I + i;
        for (int64_t k = 0; k < H; ++k)
          wrow[k] = bf16_value(bf16_nearest(grid_value(p13 + rg * (H / 2), st13 + rg * (H / 32), k)));
        for (int64_t k = 0; k < H; ++k) g = g + bf16_value(x[t * H + k]) * wrow[k];
        for (int64_t k = 0; k < H; ++k)
          wrow[k] = bf16_value(bf16_nearest(grid_value(p13 + ru * (H / 2), st13 + ru * (H / 32), k)));
        for (int64_t k = 0; k < H; ++k) u = u + bf16_value(x[t * H + k]) * wrow[k];
        const float silu = g / (1.0f + expf(-g));
        act[i] = bf16_nearest(silu * u);
        if (act16) act16[r * I + i] = act[i];
      }
      for (int64_t h = 0; h < H; ++h) {
        const int64_t rd = e * H + h;
        float acc = 0.0f;
        for (int64_t i = 0; i < I; ++i)
          acc = acc + bf16_value(act[i]) * bf16_value(bf16_nearest(grid_value(p2 + rd * (I / 2), st2 + rd * (I / 32), i)));
        d[j * H + h] = acc;
        if (d32) d32[r * H + h] = acc;
      }
    }
    for (int64_t h = 0; h < H; ++h) {
      float y = 0.0f;
      for (int j = 0; j < topk; ++j) y = y + probs[t * topk + j] * d[j * H + h];
      if (y32) y32[t * H + h] = y;
      if (y16) y16[t * H + h] = bf16_nearest(y);
    }
    free(wrow);
    free(act);
    free(d);
  }
}

int qo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the following parallel loops (timing of the benchmark's CPU
 * baseline on a given core count; no effect on any result). */
void qo_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
