/*
 * Seeded synthetic inputs for the dense prefill indexer (MQA logits + top-K).
 *
 * This file holds only random-number generation and the data quantisers that
 * turn float draws into stored fp8 / MXFP4 bytes.  It computes nothing of the
 * indexer itself (no dot products, no ReLU, no weighting, no selection): both
 * the GPU path and the CPU oracle consume the bytes it writes.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used counter-style: draw i of a stream is
 * mix(base + (i + 1) * GAMMA), where base depends on (seed, stream id).  Every
 * draw is therefore independent of thread count and evaluation order.
 * Uniforms take the top 53 bits; normals use the Box-Muller cosine branch on
 * draws (2e, 2e + 1).
 *
 * Quantisers:
 *  - fp8 E4M3 (OCP 8-bit floating point spec, "FN" variant: bias 7, max 448,
 *    no infinities, S.1111.111 is NaN): one fp32 scale per row of `cols`
 *    values, scale = amax / 448 (1 when the row is all zero); codes are
 *    round-to-nearest-even of x / scale with saturation at 448.
 *  - MXFP4 (OCP Microscaling v1.0): E2M1 elements (grid 0, .5, 1, 1.5, 2, 3,
 *    4, 6), one E8M0 scale per 32 consecutive values, shared exponent
 *    floor(log2 amax) - 2, element codes round-to-nearest-even with
 *    saturation at 6.  Two elements per byte, even index in the low nibble.
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint32_t stream) {
  return mix64(seed * 0x100000001B3ull ^ ((uint64_t)stream << 32) ^ 0xC2B2AE3D27D4EB4Full);
}

static inline uint64_t draw(uint64_t base, uint64_t i) { return mix64(base + (i + 1) * GAMMA); }

/* uniform in (0, 1): never exactly 0 or 1 */
static inline double unif(uint64_t base, uint64_t i) {
  return ((double)(draw(base, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal(uint64_t base, uint64_t e) {
  double u1 = unif(base, 2 * e), u2 = unif(base, 2 * e + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

void synth_uniform(uint64_t seed, uint32_t stream, int64_t first, int64_t n, double *out) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unif(b, (uint64_t)(first + i));
}

void synth_uniform_f32(uint64_t seed, uint32_t stream, int64_t n, float lo, float hi, float *out) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * unif(b, (uint64_t)i));
}

void synth_normal(uint64_t seed, uint32_t stream, int64_t first, int64_t n, double *out) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = normal(b, (uint64_t)(first + i));
}

void synth_u64(uint64_t seed, uint32_t stream, int64_t n, uint64_t *out) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(b, (uint64_t)i);
}

/* ---- fp8 E4M3FN encoder (round to nearest even, saturating) ---- */
static inline uint8_t enc_e4m3(double x) {
  uint8_t s = 0;
  if (x < 0) { s = 0x80; x = -x; }
  if (!(x > 0)) return 0;
  if (x > 448.0) x = 448.0;
  if (x < 0.015625) {            /* below 2^-6: subnormal grid of 2^-9 */
    double m = nearbyint(x * 512.0);   /* default rounding mode: ties to even */
    if (m == 0) return 0;
    return (uint8_t)(s | (uint8_t)m);  /* m == 8 is the code of 2^-6 */
  }
  int ex;
  double f = frexp(x, &ex);      /* x = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;                /* x = (2f) * 2^e, 2f in [1, 2) */
  double m = nearbyint((2.0 * f - 1.0) * 8.0);
  if (m == 8.0) { m = 0.0; e += 1; }
  int code = ((e + 7) << 3) | (int)m;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(s | code);
}

/* Normal draws for a [rows, cols] tensor, quantised per row to E4M3FN. */
void synth_fp8_normal_rows(uint64_t seed, uint32_t stream, int64_t rows, int32_t cols,
                           uint8_t *codes, float *scales) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double buf[1024];
    double amax = 0;
    for (int32_t c = 0; c < cols; ++c) {
      double v = normal(b, (uint64_t)(r * cols + c));
      buf[c] = v;
      double a = fabs(v);
      if (a > amax) amax = a;
    }
    float sc = amax > 0 ? (float)(amax / 448.0) : 1.0f;
    scales[r] = sc;
    for (int32_t c = 0; c < cols; ++c) codes[r * cols + c] = enc_e4m3(buf[c] / (double)sc);
  }
}

/* ---- MXFP4: E2M1 elements + E8M0 block scales ---- */
static inline uint8_t enc_e2m1(double x) {
  uint8_t s = 0;
  if (x < 0) { s = 8; x = -x; }
  /* grid 0 .5 1 1.5 2 3 4 6 (codes 0..7); ties go to the even code */
  uint8_t c;
  if (x < 0.25) c = 0;
  else if (x == 0.25) c = 0;
  else if (x < 0.75) c = 1;
  else if (x == 0.75) c = 2;
  else if (x < 1.25) c = 2;
  else if (x == 1.25) c = 2;
  else if (x < 1.75) c = 3;
  else if (x == 1.75) c = 4;
  else if (x < 2.5) c = 4;
  else if (x == 2.5) c = 4;
  else if (x < 3.5) c = 5;
  else if (x == 3.5) c = 6;
  else if (x < 5.0) c = 6;
  else if (x == 5.0) c = 6;
  else c = 7;
  if (c == 0) return 0;
  return (uint8_t)(s | c);
}

/* Normal draws for a [rows, cols] tensor (cols % 32 == 0), quantised to MXFP4.
 * packed: [rows, cols/2] bytes; e8m0: [rows, cols/32] bytes. */
void synth_mxfp4_normal_rows(uint64_t seed, uint32_t stream, int64_t rows, int32_t cols,
                             uint8_t *packed, uint8_t *e8m0) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t blk = 0; blk < cols / 32; ++blk) {
      double v[32];
      double amax = 0;
      for (int i = 0; i < 32; ++i) {
        v[i] = normal(b, (uint64_t)(r * cols + blk * 32 + i));
        double a = fabs(v[i]);
        if (a > amax) amax = a;
      }
      int E = 0;
      if (amax > 0) {
        int ex;
        frexp(amax, &ex);        /* amax in [2^(ex-1), 2^ex) */
        E = (ex - 1) - 2;
      }
      if (E < -127) E = -127;
      if (E > 127) E = 127;
      e8m0[r * (cols / 32) + blk] = (uint8_t)(E + 127);
      double inv = ldexp(1.0, -E);
      for (int i = 0; i < 32; i += 2) {
        uint8_t lo = enc_e2m1(v[i] * inv), hi = enc_e2m1(v[i + 1] * inv);
        packed[r * (cols / 2) + blk * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* Exposed encoders for the generator's own tests. */
void synth_encode_e4m3(const double *x, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = enc_e4m3(x[i]);
}
void synth_encode_e2m1(const double *x, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = enc_e2m1(x[i]);
}
