/*
 * CPU oracle for fused (Add)RmsNorm + per-row symmetric dynamic quantization,
 * the INT8 GEMM that consumes its codes, and AddLora.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * library never does.  It shares no code, header or constant table with the
 * GPU path.
 *
 * Sources (Huawei Ascend CANN operator pages):
 *  - "aclnnAddRmsNormDynamicQuantV2", Formula section: x = x1 + x2;
 *    y = x / Rms(x) * gamma + beta with Rms(x) = sqrt(mean(x^2) + epsilon);
 *    input_k = y * smoothScale_k when that smooth scale is given, else y;
 *    scale_kOut = row_max(|input_k|) / 127 (INT8) or / 7 (INT4);
 *    y_kOut = round(input_k / scale_kOut); the output-validity cases, and
 *    the Constraints section's rules on outputMask and the smooth scales.
 *  - "aclnnRmsNormDynamicQuant", formula section (计算公式): the single-input
 *    form (no add, one output, optional smoothScales, max_val 127 for INT8).
 *  - "aclnnAddLora", Formulas: grouped shrink / expand and slice-accumulate
 *    (readings listed at oracle_add_lora below).
 *  - The INT8 GEMM that consumes the quantized rows is not on the pages; it
 *    is defined from the V2 Formula (see oracle_w8a8_gemm_at).
 *
 * Readings taken where the pages are silent (each one is also listed in the
 * design notes of the repository):
 *  - arithmetic is real-valued: this oracle works in double throughout and
 *    rounds only what is stored (xOut to the input type, scales to float);
 *  - the norm uses the unrounded sum x1 + x2, not the stored xOut;
 *  - round() is round-half-to-even; codes are clamped to [-Q, Q];
 *  - the code is round(input / scale) with the scale as stored (float);
 *  - a stored scale of 0 (row max 0) gives all-zero codes;
 *  - epsilon is applied as the float nearest to the given value;
 *  - beta absent means beta = 0; a smooth scale absent means factor 1;
 *  - with outputMask absent and neither smooth scale given, the second
 *    output is not produced (the pages' case list covers neither branch).
 *
 * Build: gcc -O2 -fPIC -shared adq_oracle.c -o libadq_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_F16 1

/* --- storage types ------------------------------------------------------ */

/* Exact value of a bfloat16 bit pattern: sign, 8-bit exponent (bias 127),
 * 7-bit fraction; exponent 0 means subnormal with scale 2^-133. */
static double bf16_value(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xFF;
  int f = b & 0x7F;
  double v;
  if (e == 0xFF) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -133);
  else v = ldexp((double)(128 + f), e - 134);
  return sign ? -v : v;
}

/* Exact value of an IEEE binary16 bit pattern: 5-bit exponent (bias 15),
 * 10-bit fraction; exponent 0 means subnormal with scale 2^-24. */
static double f16_value(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0x1F) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -24);
  else v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

double oracle_storage_value(uint16_t bits, int dtype) {
  return dtype == ORACLE_BF16 ? bf16_value(bits) : f16_value(bits);
}

/*
 * Round a double to the nearest value of the storage type, ties to even,
 * and return its bit pattern.  Written from the definition: find the
 * quantum (spacing of representable values) at |a|, divide, round the
 * quotient to the nearest even integer, multiply back.  Results at or above
 * 2^(emax+1) overflow to infinity, as round-to-nearest does.
 */
uint16_t oracle_round_to_storage(double a, int dtype) {
  const int p = dtype == ORACLE_BF16 ? 8 : 11;       /* significand bits */
  const int emin = dtype == ORACLE_BF16 ? -126 : -14; /* smallest normal exponent */
  const int emax = dtype == ORACLE_BF16 ? 127 : 15;
  const int ebits_bias = dtype == ORACLE_BF16 ? 127 : 15;
  uint16_t sign = signbit(a) ? 0x8000u : 0u;
  double m = fabs(a);
  if (isnan(a)) return (uint16_t)(dtype == ORACLE_BF16 ? 0x7FC0u : 0x7E00u);
  uint16_t inf = (uint16_t)(dtype == ORACLE_BF16 ? 0x7F80u : 0x7C00u);
  if (isinf(a)) return (uint16_t)(sign | inf);
  if (m == 0.0) return sign;
  int ex;
  frexp(m, &ex); /* m = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;  /* m in [2^e, 2^(e+1)) */
  if (e < emin) e = emin;
  double quantum = ldexp(1.0, e - (p - 1));
  double q = nearbyint(m / quantum); /* default FE_TONEAREST: ties to even */
  double r = q * quantum;
  if (r >= ldexp(1.0, emax + 1)) return (uint16_t)(sign | inf);
  if (r < ldexp(1.0, emin)) {
    /* subnormal: fraction field holds r / 2^(emin - p + 1) */
    return (uint16_t)(sign | (uint16_t)q);
  }
  int er;
  frexp(r, &er);
  int eu = er - 1; /* r in [2^eu, 2^(eu+1)) */
  uint32_t frac = (uint32_t)(ldexp(r, (p - 1) - eu) - ldexp(1.0, p - 1));
  uint32_t bits = ((uint32_t)(eu + ebits_bias) << (p - 1)) | frac;
  return (uint16_t)(sign | bits);
}

/* --- which outputs exist ------------------------------------------------ */

/*
 * Output validity, "aclnnAddRmsNormDynamicQuantV2" Formula (the cases of
 * scale1Out/y1Out/scale2Out/y2Out) and Constraints (mask rules).
 * mask: NULL when outputMaskOptional is absent, else two flags.
 * Returns 1 and sets act1/act2 for a legal call, 0 for a call the
 * Constraints section forbids.
 */
int oracle_v2_outputs(const int* mask, int has_s1, int has_s2, int* act1, int* act2) {
  if (mask) {
    if (has_s1 && !mask[0]) return 0; /* smooth1 given needs mask[0] */
    if (has_s2 && !mask[1]) return 0; /* smooth2 given needs mask[1] */
    if (!mask[0] && !mask[1]) return 0; /* both false is forbidden */
    *act1 = mask[0] ? 1 : 0;
    *act2 = mask[1] ? 1 : 0;
    return 1;
  }
  if (has_s2 && !has_s1) return 0; /* mask absent: smooth2 needs smooth1 */
  *act1 = 1;                       /* mask absent: the first output always exists */
  *act2 = (has_s1 && has_s2) ? 1 : 0;
  return 1;
}

/* --- the row computation ------------------------------------------------ */

/*
 * rows x n inputs, row-major, 16-bit storage of type dtype.
 * x2 == NULL selects the single-input RmsNormDynamicQuant form (x = x1).
 * q1, q2: the quantization maximum of each output (127 for INT8, 7 for
 * INT4) or 0 when that output is not produced.
 * Outputs (each may be NULL when not wanted):
 *   x_out   [rows, n]  storage type, the rounded sum x1 + x2;
 *   code_k  [rows, n]  int8 codes (INT4 codes unpacked, one per byte);
 *   scale_k [rows]     float scales;
 *   pre_k   [rows, n]  double input_k / scale_k before rounding.
 * Returns 0, or -1 for bad arguments.
 */
int oracle_add_rms_norm_dq(int64_t rows, int64_t n, int dtype, const uint16_t* x1,
                           const uint16_t* x2, const uint16_t* gamma, const uint16_t* beta,
                           const uint16_t* smooth1, const uint16_t* smooth2, double epsilon,
                           int q1, int q2, uint16_t* x_out, int8_t* code1, int8_t* code2,
                           float* scale1, float* scale2, double* pre1, double* pre2,
                           double* work /* 2 * n doubles */) {
  if (rows < 0 || n <= 0 || !x1 || !gamma || !work) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return -1;
  const double eps = (double)(float)epsilon;
  double* a = work;     /* x = x1 + x2, unrounded */
  double* y = work + n; /* RmsNorm output */
  const int qk[2] = {q1, q2};
  const uint16_t* smooth[2] = {smooth1, smooth2};
  int8_t* codes[2] = {code1, code2};
  float* scales[2] = {scale1, scale2};
  double* pres[2] = {pre1, pre2};

  for (int64_t i = 0; i < rows; ++i) {
    const int64_t off = i * n;
    /* x = x1 + x2 (V2 Formula, first equation), exact in double for all
     * pairs whose exponents are within 44 binades of each other. */
    for (int64_t j = 0; j < n; ++j) {
      double v = oracle_storage_value(x1[off + j], dtype);
      if (x2) v += oracle_storage_value(x2[off + j], dtype);
      a[j] = v;
      if (x_out) x_out[off + j] = oracle_round_to_storage(v, dtype);
    }
    /* Rms(x) = sqrt(1/n * sum x_j^2 + epsilon) (RmsNorm equation). */
    double ss = 0.0;
    for (int64_t j = 0; j < n; ++j) ss += a[j] * a[j];
    const double rms = sqrt(ss / (double)n + eps);
    /* y = x / Rms(x) * gamma + beta. */
    for (int64_t j = 0; j < n; ++j) {
      double g = oracle_storage_value(gamma[j], dtype);
      double b = beta ? oracle_storage_value(beta[j], dtype) : 0.0;
      y[j] = a[j] / rms * g + b;
    }
    for (int k = 0; k < 2; ++k) {
      if (qk[k] == 0) continue;
      const double Q = (double)qk[k];
      /* input_k = y * smoothScale_k, or y when absent; row_max(|input_k|). */
      double m = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        double in = smooth[k] ? y[j] * oracle_storage_value(smooth[k][j], dtype) : y[j];
        if (fabs(in) > m) m = fabs(in);
      }
      /* scale_k = row_max / Q, stored as float. */
      const float sc = (float)(m / Q);
      if (scales[k]) scales[k][i] = sc;
      /* y_k = round(input_k / scale_k), half to even, within [-Q, Q]. */
      for (int64_t j = 0; j < n; ++j) {
        double in = smooth[k] ? y[j] * oracle_storage_value(smooth[k][j], dtype) : y[j];
        double v = (sc == 0.0f) ? 0.0 : in / (double)sc;
        double c = nearbyint(v);
        if (c > Q) c = Q;
        if (c < -Q) c = -Q;
        if (codes[k]) codes[k][off + j] = (int8_t)c;
        if (pres[k]) pres[k][off + j] = v;
      }
    }
  }
  return 0;
}

/*
 * INT4 storage: two codes per byte, the even column in the low nibble and
 * the odd column in the high nibble, each as a 4-bit two's complement
 * value.  codes [rows, n] int8 in [-8, 7], n even; out [rows, n/2].
 */
int oracle_pack_int4(int64_t rows, int64_t n, const int8_t* codes, uint8_t* out) {
  if (n % 2 != 0 || !codes || !out) return -1;
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < n / 2; ++j) {
      uint8_t lo = (uint8_t)codes[i * n + 2 * j] & 0x0Fu;
      uint8_t hi = (uint8_t)codes[i * n + 2 * j + 1] & 0x0Fu;
      out[i * (n / 2) + j] = (uint8_t)(lo | (hi << 4));
    }
  return 0;
}

/* --- the consumer of the codes: INT8 x INT8 GEMM with scales ------------- */

/*
 * With y1Out = round(input1 / scale1Out) ("aclnnAddRmsNormDynamicQuantV2",
 * Formula), input1 is approximated by y1Out * scale1Out row by row; a linear
 * layer with per-output-column weight scales then computes, for each
 * requested output (row mi[t], column ni[t]):
 *   sums[t] = sum_k a[mi[t], k] * w[ni[t], k]          (exact, int64)
 *   out[t]  = sums[t] * a_scale[mi[t]] * w_scale[ni[t]] + bias[ni[t]]   (double)
 * a is [rows, k] and w is [n, k], both row-major int8; bias may be NULL.
 */
int oracle_w8a8_gemm_at(int64_t count, const int64_t* mi, const int64_t* ni, int64_t k,
                        const int8_t* a, const float* a_scale, const int8_t* w,
                        const float* w_scale, const float* bias, int64_t* sums, double* out) {
  if (count < 0 || k <= 0 || !mi || !ni || !a || !a_scale || !w || !w_scale) return -1;
  for (int64_t t = 0; t < count; ++t) {
    const int8_t* ar = a + mi[t] * k;
    const int8_t* wr = w + ni[t] * k;
    int64_t s = 0;
    for (int64_t j = 0; j < k; ++j) s += (int64_t)ar[j] * (int64_t)wr[j];
    if (sums) sums[t] = s;
    if (out)
      out[t] = (double)s * (double)a_scale[mi[t]] * (double)w_scale[ni[t]] +
               (bias ? (double)bias[ni[t]] : 0.0);
  }
  return 0;
}

/* --- AddLora ------------------------------------------------------------- */

/*
 * "aclnnAddLora", Formulas: rows of x are grouped by their index in
 * `indices`; for each group i the shrink Z1 = x_i . weightA[i, layerIdx]
 * and the expand Z2 = Z1 . weightB[i, layerIdx] x scale are formed, and the
 * result is accumulated into the slice y[:, yOffset : yOffset + ySliceSize]
 * to give out.  Grouping only batches rows that share weights; row by row
 * the definition is, for a row b with group g = indices[b]:
 *   Z1[r]  = sum_k x[b, k] * A[g, layer, k, r]      (A is [W, L, h1, rank])
 *   Z2[j]  = (sum_r Z1[r] * B[g, layer, r, j]) * scale   (B is [W, L, rank, h2])
 *   out[b, y_offset + j] = y[b, y_offset + j] + Z2[j],  j < h2
 *   out[b, c] = y[b, c] for every other column c of the h3-wide row.
 * Readings taken where the page is silent (its parameter tables are lost):
 *  - weightA absent: the shrink is skipped and Z1 = x[b, :] (h1 == rank);
 *  - a row whose index lies outside [0, W) gets no contribution (out = y);
 *  - arithmetic is real-valued: double throughout, out rounded once to the
 *    storage type; scale is applied as the float nearest the given value.
 * Rows to compute: rows[0 .. count) (all `nrows` rows when rows is NULL).
 * `pre` (optional, [count, h2]) receives the slice values before rounding.
 * `work` holds rank doubles.
 */
int oracle_add_lora(int64_t nrows, int64_t h1, int64_t rank, int64_t h2, int64_t h3, int64_t w,
                    int64_t l, int dtype, const uint16_t* y, const uint16_t* x,
                    const uint16_t* wa, const uint16_t* wb, const int32_t* indices,
                    int64_t layer, double scale, int64_t y_offset, int64_t count,
                    const int64_t* rows, uint16_t* out, double* pre, double* work) {
  if (nrows <= 0 || h1 <= 0 || rank <= 0 || h2 <= 0 || h3 <= 0 || w <= 0 || l <= 0) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return -1;
  if (!y || !x || !wb || !indices || !out || !work) return -1;
  if (layer < 0 || layer >= l || y_offset < 0 || y_offset + h2 > h3) return -1;
  if (!wa && h1 != rank) return -1;
  const double s = (double)(float)scale;
  const int64_t n = rows ? count : nrows;
  for (int64_t t = 0; t < n; ++t) {
    const int64_t b = rows ? rows[t] : t;
    if (b < 0 || b >= nrows) return -1;
    const uint16_t* yr = y + b * h3;
    uint16_t* o = out + t * h3;
    for (int64_t c = 0; c < h3; ++c) o[c] = yr[c];
    const int64_t g = indices[b];
    const int valid = g >= 0 && g < w;
    if (valid) {
      const uint16_t* xr = x + b * h1;
      for (int64_t r = 0; r < rank; ++r) {
        double z = 0.0;
        if (wa) {
          const uint16_t* a = wa + ((g * l + layer) * h1) * rank;
          for (int64_t k = 0; k < h1; ++k)
            z += oracle_storage_value(xr[k], dtype) * oracle_storage_value(a[k * rank + r], dtype);
        } else {
          z = oracle_storage_value(xr[r], dtype);
        }
        work[r] = z;
      }
    }
    const uint16_t* bm = valid ? wb + ((g * l + layer) * rank) * h2 : NULL;
    for (int64_t j = 0; j < h2; ++j) {
      double v = oracle_storage_value(yr[y_offset + j], dtype);
      if (valid) {
        double z2 = 0.0;
        for (int64_t r = 0; r < rank; ++r) z2 += work[r] * oracle_storage_value(bm[r * h2 + j], dtype);
        v += z2 * s;
        o[y_offset + j] = oracle_round_to_storage(v, dtype);
      }
      if (pre) pre[t * h2 + j] = v;
    }
  }
  return 0;
}
