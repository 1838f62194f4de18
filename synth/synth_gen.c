/*
 * Seeded, counter-based synthetic input generator.
 *
 * Test and benchmark infrastructure only: it produces the input tensors
 * (x1, x2, gamma, beta, smooth scales) that both the CPU oracle and the
 * GPU library consume.  It holds none of the operator's arithmetic.
 *
 * Every value is a pure function of (seed, tensor_id, flat_index), so any
 * subset of rows can be regenerated on its own and the result does not
 * depend on the number of threads.
 *
 * Draws:    d(seed, tid, i) = mix(base(seed, tid) + i * 0x9E3779B97F4A7C15)
 *           where mix is the SplitMix64 output finaliser (Steele, Lea and
 *           Flood, "Fast splittable pseudorandom number generators",
 *           OOPSLA 2014) and base(seed, tid) = mix(mix(seed) ^ tid * K).
 * Uniform:  u = (d >> 11) * 2^-53  in [0, 1).
 * Normal:   Box-Muller (cosine branch) on draws 2i and 2i+1, computed in
 *           double: z = sqrt(-2 ln(1 - u0)) * cos(2 pi u1).
 * Storage:  each double value (after any outlier factor) is rounded once,
 *           directly to the 16-bit storage type, to nearest with ties to
 *           even (no intermediate float).  Only the stored 16-bit patterns
 *           matter to the consumers.
 *
 * Build:  gcc -O2 -fPIC -shared -pthread synth_gen.c -o libsynth_gen.so -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_BF16 0
#define SYNTH_F16 1

#define SYNTH_NORMAL 0
#define SYNTH_UNIFORM 1

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint32_t tid) {
  return mix64(mix64(seed + 0x9E3779B97F4A7C15ULL) ^
               ((uint64_t)(tid + 1) * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t draw(uint64_t base, uint64_t i) {
  return mix64(base + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double unit_double(uint64_t d) {
  return (double)(d >> 11) * (1.0 / 9007199254740992.0);
}

/*
 * Round a finite double to the nearest value of a binary format with
 * `digits` significant bits, smallest normal exponent `emin` (the format's
 * normal values lie in [2^emin, 2^(emax+1))) and largest finite value
 * `maxval`; ties to even (nearbyint under the default rounding mode).  The
 * value is cut at the format's spacing at |v| (2^(e - digits + 1) for
 * |v| in [2^e, 2^(e+1)), or the subnormal spacing 2^(emin - digits + 1)),
 * scaled to an integer count of that spacing, rounded, and scaled back:
 * every step but the rounding is exact.  Values that round beyond maxval
 * become infinite.
 */
static double round_to_format(double v, int digits, int emin, double maxval) {
  if (v == 0.0) return v;
  int e;
  (void)frexp(v, &e); /* |v| in [2^(e-1), 2^e) */
  int exp = e - 1;
  if (exp < emin) exp = emin;
  const double spacing = ldexp(1.0, exp - digits + 1);
  const double r = nearbyint(v / spacing) * spacing;
  if (fabs(r) > maxval) return r > 0 ? INFINITY : -INFINITY;
  return r;
}

/* Bits of a float that is exactly a bfloat16 value (top half). */
static uint16_t bf16_bits_exact(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* Bits of a float that is exactly a binary16 value (or infinite). */
static uint16_t f16_bits_exact(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t exp = (u >> 23) & 0xFFu;
  const uint32_t man = u & 0x7FFFFFu;
  if (exp == 0xFFu) return (uint16_t)(sign | 0x7C00u);
  if (exp == 0 && man == 0) return sign;
  const int e = (int)exp - 127;
  if (e < -14) /* subnormal binary16: value = q * 2^-24 */
    return (uint16_t)(sign | (uint32_t)ldexp(fabs((double)f), 24));
  return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (man >> 13));
}

/* bfloat16: 8 significant bits, normals from 2^-126, largest (2 - 2^-7) 2^127.
 * binary16: 11 significant bits, normals from 2^-14, largest 65504. */
static inline uint16_t to_storage(double v, int dtype) {
  if (dtype == SYNTH_BF16)
    return bf16_bits_exact((float)round_to_format(v, 8, -126, 0x1.FEp127));
  return f16_bits_exact((float)round_to_format(v, 11, -14, 65504.0));
}

static inline double sample(uint64_t base, uint64_t idx, int dist, double p0, double p1) {
  if (dist == SYNTH_UNIFORM) return p0 + (p1 - p0) * unit_double(draw(base, idx));
  double u0 = unit_double(draw(base, 2 * idx));
  double u1 = unit_double(draw(base, 2 * idx + 1));
  double z = sqrt(-2.0 * log(1.0 - u0)) * cos(6.283185307179586 * u1);
  return p0 + p1 * z;
}

typedef struct {
  uint64_t base;
  int dist;
  double p0, p1;
  int dtype;
  int64_t cols;
  int64_t row0, nrows, row_offset;
  const uint8_t* outlier; /* per-column flag, may be NULL */
  double factor;
  uint16_t* out;
} fill_job;

static void fill_rows(const fill_job* j) {
  for (int64_t r = j->row0; r < j->row0 + j->nrows; ++r) {
    uint64_t flat = (uint64_t)(r + j->row_offset) * (uint64_t)j->cols;
    uint16_t* dst = j->out + r * j->cols;
    for (int64_t c = 0; c < j->cols; ++c) {
      double v = sample(j->base, flat + (uint64_t)c, j->dist, j->p0, j->p1);
      if (j->outlier && j->outlier[c]) v *= j->factor;
      dst[c] = to_storage(v, j->dtype);
    }
  }
}

static void* fill_thread(void* arg) {
  fill_rows((const fill_job*)arg);
  return NULL;
}

/*
 * Fill out[rows, cols] with the values of rows [row_offset, row_offset+rows)
 * of the tensor (seed, tid).  dist: 0 = normal(mean p0, std p1),
 * 1 = uniform[p0, p1).  outlier: optional per-column 0/1 flags; flagged
 * columns are multiplied by factor before storage rounding.
 */
int synth_fill(uint64_t seed, uint32_t tid, int dist, double p0, double p1, int dtype,
               int64_t rows, int64_t cols, int64_t row_offset, const uint8_t* outlier,
               double factor, int nthreads, uint16_t* out) {
  if (rows < 0 || cols < 0 || !out) return -1;
  if (dtype != SYNTH_BF16 && dtype != SYNTH_F16) return -1;
  if (dist != SYNTH_NORMAL && dist != SYNTH_UNIFORM) return -1;
  uint64_t base = stream_base(seed, tid);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if ((int64_t)nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
  fill_job jobs[64];
  pthread_t th[64];
  int64_t per = rows / nthreads, extra = rows % nthreads, r0 = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t n = per + (t < extra ? 1 : 0);
    fill_job j = {base, dist, p0, p1, dtype, cols, r0, n, row_offset, outlier, factor, out};
    jobs[t] = j;
    r0 += n;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, fill_thread, &jobs[t]) != 0) break;
    started = t;
  }
  fill_rows(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; ++t) fill_rows(&jobs[t]);
  return 0;
}

/*
 * Choose k distinct columns out of n with a seeded partial Fisher-Yates
 * shuffle (draw i picks position i + d mod (n - i)); flags[c] = 1 for the
 * chosen columns.
 */
int synth_pick_columns(uint64_t seed, uint32_t tid, int64_t n, int64_t k, int64_t* scratch,
                       uint8_t* flags) {
  if (k < 0 || k > n || !scratch || !flags) return -1;
  uint64_t base = stream_base(seed, tid);
  for (int64_t i = 0; i < n; ++i) {
    scratch[i] = i;
    flags[i] = 0;
  }
  for (int64_t i = 0; i < k; ++i) {
    int64_t j = i + (int64_t)(draw(base, (uint64_t)i) % (uint64_t)(n - i));
    int64_t t = scratch[i];
    scratch[i] = scratch[j];
    scratch[j] = t;
    flags[scratch[i]] = 1;
  }
  return 0;
}

/*
 * Uniform integers in [lo, hi] as int8 (rows [row_offset, row_offset+rows)
 * of the tensor (seed, tid), cols per row): draw modulo (hi - lo + 1).
 */
int synth_fill_int8(uint64_t seed, uint32_t tid, int lo, int hi, int64_t rows, int64_t cols,
                    int64_t row_offset, int8_t* out) {
  if (rows < 0 || cols < 0 || !out || lo > hi || lo < -128 || hi > 127) return -1;
  uint64_t base = stream_base(seed, tid);
  uint64_t span = (uint64_t)(hi - lo + 1);
  for (int64_t r = 0; r < rows; ++r) {
    uint64_t flat = (uint64_t)(r + row_offset) * (uint64_t)cols;
    for (int64_t c = 0; c < cols; ++c)
      out[r * cols + c] = (int8_t)(lo + (int)(draw(base, flat + (uint64_t)c) % span));
  }
  return 0;
}

/* n float32 values of the tensor (seed, tid): dist 0 normal(p0, p1), 1 uniform[p0, p1). */
int synth_fill_f32(uint64_t seed, uint32_t tid, int dist, double p0, double p1, int64_t n,
                   float* out) {
  if (n < 0 || !out) return -1;
  uint64_t base = stream_base(seed, tid);
  for (int64_t i = 0; i < n; ++i) out[i] = (float)sample(base, (uint64_t)i, dist, p0, p1);
  return 0;
}

/* n int32 values of the tensor (seed, tid), uniform in [lo, hi] (draw modulo hi - lo + 1). */
int synth_fill_i32(uint64_t seed, uint32_t tid, int64_t lo, int64_t hi, int64_t n, int32_t* out) {
  if (n < 0 || !out || lo > hi || lo < INT32_MIN || hi > INT32_MAX) return -1;
  uint64_t base = stream_base(seed, tid);
  uint64_t span = (uint64_t)(hi - lo + 1);
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)(lo + (int64_t)(draw(base, (uint64_t)i) % span));
  return 0;
}
