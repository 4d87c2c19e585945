/*
 * CPU oracle of the dense prefill indexer -- TEST INFRASTRUCTURE.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library (through oracle/__init__.py).  The indexer library itself
 * never does: it runs its HIP kernels or fails.  Nothing here is shared with
 * the HIP library (no kernels, headers, helpers, tables or constants); this
 * file reads only the bytes the seeded generator writes.
 *
 * Plain single-threaded C++ in fp64: every function is the definition written
 * out, with std::sort as the only library primitive.  There is no blocking,
 * fusion or reordering.  Callers that want several rows at once run this
 * code on several threads, one row per call.
 *
 * Sources (web pages, cited by title and section):
 *   P1  "Running CHUNKED_PREFILL_SIZE above 1024 without the long-prompt
 *       memory problem": section 1 (the dense indexer call: a chunk's rows
 *       scored against the whole compressed prefix, logits [T, max_seqlen_k]
 *       fp32, a ragged top-k, and the layer that pools 8-key blocks, keeps the
 *       top-2048 blocks and publishes a bool mask applied by masked_fill_),
 *       section 2.1 (a request landing on a cached prefix), section 2.3 (key
 *       blocks with per-block top-k and a merge).
 *   P2  "[DeepSeek-V4.1] Bound the dense prefill indexer transient: row-chunk
 *       logits, tail-only candidate masks": Motivation (fp8 queries x fp4 keys,
 *       logits [T, lc] fp32), Accuracy/equivalence (index sets and masks are
 *       compared; ties among repeated keys are the only residual).
 *
 * The score formula is not printed on the pages.  The oracle uses the
 * DeepSeek sparse-attention indexer score: for query row t and key s in the
 * row's window [ks_t, ke_t),
 *
 *     I[t, s] = sum_h w[t, h] * max(0, scale * sum_d qd[t, h, d] * kd[s, d])
 *
 * with qd, kd the dequantised fp8 / MXFP4 inputs.  Readings where the pages are
 * silent: q has one fp32 scale per (t, h) row of D values, fp8 keys one per key
 * row, MXFP4 keys one E8M0 scale per 32 consecutive d; outside the window the
 * logit is -inf; the top-k decision is taken on the fp32 rounding of the score
 * (the pages' logits dtype), ordered by (value desc, key index asc); selected
 * keys are listed ascending, padded with -1; pooling blocks of 8 keys start at
 * ks_t and a partial last block takes the max of its in-window keys.
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <vector>

namespace {

const double NEG_INF = -std::numeric_limits<double>::infinity();
const double NOT_A_NUMBER = std::numeric_limits<double>::quiet_NaN();

// OCP "8-bit Floating Point Specification (OFP8)", E4M3 ("FN": no infinities):
// sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.  Exponent
// field 0 is subnormal, m/8 * 2^(1 - 7); S.1111.111 is NaN; largest value 448.
double e4m3(uint32_t c) {
  const double sign = (c & 0x80u) ? -1.0 : 1.0;
  const int e = (int)((c >> 3) & 0xFu);
  const int m = (int)(c & 0x7u);
  if (e == 15 && m == 7) return NOT_A_NUMBER;
  if (e == 0) return sign * std::ldexp((double)m / 8.0, 1 - 7);
  return sign * std::ldexp(1.0 + (double)m / 8.0, e - 7);
}

// OCP "Microscaling Formats (MX) v1.0", FP4 E2M1 element: sign bit 3,
// exponent bits 2..1 with bias 1, mantissa bit 0; exponent field 0 is
// subnormal, m/2 * 2^(1 - 1); no infinities or NaN.
double e2m1(uint32_t c) {
  const double sign = (c & 0x8u) ? -1.0 : 1.0;
  const int e = (int)((c >> 1) & 0x3u);
  const int m = (int)(c & 0x1u);
  if (e == 0) return sign * ((double)m / 2.0);
  return sign * std::ldexp(1.0 + (double)m / 2.0, e - 1);
}

// OCP MX v1.0 E8M0 scale: 2^(c - 127); code 255 is NaN.
double e8m0(uint32_t c) {
  if (c == 255u) return NOT_A_NUMBER;
  return std::ldexp(1.0, (int)c - 127);
}

// The fp32 number the pages' logits dtype holds for an fp64 score.
float as_fp32(double v) { return (float)v; }

}  // namespace

extern "C" {

// ---------------------------------------------------------------- decoders
void orc_decode_e4m3(const uint8_t *codes, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3(codes[i]);
}
void orc_decode_e2m1(const uint8_t *codes, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e2m1(codes[i] & 0xFu);
}
void orc_decode_e8m0(const uint8_t *codes, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e8m0(codes[i]);
}

// qd[t, h, d] = e4m3(q8[t, h, d]) * q_scale[t, h] for rows [t0, t1) (out: [t1 - t0, H, D]).
void orc_dequant_q(const uint8_t *q, const float *q_scale, int64_t t0, int64_t t1, int32_t H, int32_t D,
                   double *out) {
  for (int64_t t = t0; t < t1; ++t)
    for (int32_t h = 0; h < H; ++h)
      for (int32_t d = 0; d < D; ++d)
        out[((t - t0) * H + h) * D + d] = e4m3(q[(t * H + h) * D + d]) * (double)q_scale[t * H + h];
}

// kd[s, d] for every key row: fp8 keys e4m3(k8[s, d]) * k_scale[s]; MXFP4 keys
// e2m1(element d) * e8m0(k_scale[s, d / 32]), element d in the low nibble of
// byte d / 2 when d is even (P2 Motivation: fp8 queries x fp4 keys).
// Returns 0, or -1 for an unknown format.
int32_t orc_dequant_k(const uint8_t *k, const void *k_scale, int32_t k_fmt, int64_t L, int32_t D, double *kd) {
  if (k_fmt == 0) {
    const float *sc = (const float *)k_scale;
    for (int64_t s = 0; s < L; ++s)
      for (int32_t d = 0; d < D; ++d) kd[s * D + d] = e4m3(k[s * D + d]) * (double)sc[s];
    return 0;
  }
  if (k_fmt == 1) {
    const uint8_t *e8 = (const uint8_t *)k_scale;
    for (int64_t s = 0; s < L; ++s)
      for (int32_t d = 0; d < D; ++d) {
        const uint8_t byte = k[s * (D / 2) + d / 2];
        const uint32_t nib = (d % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
        kd[s * D + d] = e2m1(nib) * e8m0(e8[s * (D / 32) + d / 32]);
      }
    return 0;
  }
  return -1;
}

// ---------------------------------------------------------------- logits
// I[t, s] for the keys s of [ks, ke), written to out[s - ks] (P1 section 1: every
// query row of the chunk is scored against its whole key window).  q: E4M3 codes
// [T, H, D]; kd: dequantised keys [L, D].  Each head's dot runs over d in order;
// heads are summed in order.  Returns 0, or -1 when the window is not inside [0, L].
int32_t orc_row_logits(const uint8_t *q, const float *q_scale, const float *w, int32_t H, int32_t D,
                       const double *kd, int64_t L, int64_t t, int64_t ks, int64_t ke, double scale, double *out) {
  if (ks < 0 || ke < ks || ke > L) return -1;
  // this row's dequantised queries, stored d-major so that the heads' sums sit side by side
  std::vector<double> qd((size_t)D * H), wt((size_t)H), dot((size_t)H);
  for (int32_t h = 0; h < H; ++h) {
    wt[h] = (double)w[t * H + h];
    for (int32_t d = 0; d < D; ++d)
      qd[(size_t)d * H + h] = e4m3(q[(t * H + h) * D + d]) * (double)q_scale[t * H + h];
  }
  for (int64_t s = ks; s < ke; ++s) {
    const double *kv = kd + s * D;
    for (int32_t h = 0; h < H; ++h) dot[h] = 0.0;
    for (int32_t d = 0; d < D; ++d) {
      const double kval = kv[d];
      const double *qrow = &qd[(size_t)d * H];
      for (int32_t h = 0; h < H; ++h) dot[h] += qrow[h] * kval;
    }
    double acc = 0.0;
    for (int32_t h = 0; h < H; ++h) {
      const double x = scale * dot[h];
      acc += wt[h] * (x > 0.0 ? x : 0.0);
    }
    out[s - ks] = acc;
  }
  return 0;
}

// ---------------------------------------------------------------- selection
// Top-K of one row's window (P1 section 2.3, P2 Modifications: a ragged top-k per
// row).  vals: fp64 logits, index j <-> key ks + j.  allowed (nullable): keys with
// allowed[j] == 0 are excluded (the candidate mask: masked_fill_ with -inf, never
// selected).  Order: fp32 value desc, then index asc.  idx: [K] selected keys
// ascending, then -1; val: their fp32 values, then -inf.
void orc_topk_row(const double *vals, int64_t n, const uint8_t *allowed, int64_t ks, int32_t K, int32_t *idx,
                  float *val) {
  std::vector<int64_t> pos;
  pos.reserve((size_t)n);
  for (int64_t j = 0; j < n; ++j)
    if (!allowed || allowed[j]) pos.push_back(j);
  std::sort(pos.begin(), pos.end(), [&](int64_t a, int64_t b) {
    const float va = as_fp32(vals[a]), vb = as_fp32(vals[b]);
    if (va != vb) return va > vb;
    return a < b;
  });
  const size_t take = std::min(pos.size(), (size_t)(K > 0 ? K : 0));
  std::vector<int64_t> sel(pos.begin(), pos.begin() + (int64_t)take);
  std::sort(sel.begin(), sel.end());
  for (int32_t i = 0; i < K; ++i) {
    if ((size_t)i < take) {
      idx[i] = (int32_t)(ks + sel[i]);
      val[i] = as_fp32(vals[sel[i]]);
    } else {
      idx[i] = -1;
      val[i] = -std::numeric_limits<float>::infinity();
    }
  }
}

// P[b] = max of vals over j in [pool b, pool b + pool) inside [0, n) (P1 section 1:
// the logits are padded with -inf and pooled over blocks of `pool` keys from ks, so a
// partial last block takes the max of its valid keys).  out: [ceil(n / pool)].
void orc_pool_row(const double *vals, int64_t n, int32_t pool, double *out) {
  const int64_t nb = (n + pool - 1) / pool;
  for (int64_t b = 0; b < nb; ++b) {
    double m = NEG_INF;
    for (int64_t j = b * pool; j < std::min((b + 1) * pool, n); ++j) m = std::max(m, vals[j]);
    out[b] = m;
  }
}

// Candidate source of one row (P1 section 1): pool, keep the n_blocks blocks with the
// largest pooled fp32 value (ties: lower block), mask[j] = 1 for j < W iff j < n and
// block j / pool is kept.  chosen: [min(n_blocks, blocks)] kept blocks ascending.
// Returns the number of kept blocks.
int32_t orc_block_candidates_row(const double *vals, int64_t n, int32_t pool, int32_t n_blocks, int64_t W,
                                 uint8_t *mask, int32_t *chosen) {
  const int64_t nb = (n + pool - 1) / pool;
  std::vector<double> P((size_t)nb);
  orc_pool_row(vals, n, pool, P.data());
  std::vector<int64_t> order((size_t)nb);
  for (int64_t b = 0; b < nb; ++b) order[b] = b;
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    const float va = as_fp32(P[a]), vb = as_fp32(P[b]);
    if (va != vb) return va > vb;
    return a < b;
  });
  const int64_t take = std::min<int64_t>(nb, n_blocks);
  std::vector<int64_t> sel(order.begin(), order.begin() + take);
  std::sort(sel.begin(), sel.end());
  for (int64_t j = 0; j < W; ++j) mask[j] = 0;
  for (int64_t i = 0; i < take; ++i) {
    chosen[i] = (int32_t)sel[i];
    for (int64_t j = sel[i] * pool; j < std::min((sel[i] + 1) * pool, n); ++j)
      if (j < W) mask[j] = 1;
  }
  return (int32_t)take;
}

// ---------------------------------------------------------------- windows
// Per-row key windows [ks, ke) of a varlen batch, row by row.  Request i owns query
// rows [cu_q[i], cu_q[i+1]) and token rows [cu_k[i], cu_k[i+1]); its len_q new tokens
// are the last of its len_k tokens (P1 section 2.1: a request may land on a cached
// prefix), so new row j is token prefix + j, prefix = len_k - len_q, and has seen
// prefix + j + 1 tokens (P1 section 1: a row's window runs up to its own position).
// Keys are one per `ratio` consecutive tokens, in rows [cu_c[i], cu_c[i+1]) (P1
// section 1: the ratio-1/2 layers score against the compressed prefix); a row sees the
// keys of its complete groups, floor(seen / ratio), at most the request's key count.
// Reading: the pages give the compressed length, not how a partial group counts; a key
// summarises a whole group, so it becomes visible once its group is complete.
void orc_ragged_windows(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_c, int32_t B, int32_t ratio,
                        int32_t *ks, int32_t *ke) {
  for (int32_t i = 0; i < B; ++i) {
    const int64_t len_q = (int64_t)cu_q[i + 1] - cu_q[i];
    const int64_t len_k = (int64_t)cu_k[i + 1] - cu_k[i];
    const int64_t len_c = (int64_t)cu_c[i + 1] - cu_c[i];
    for (int64_t j = 0; j < len_q; ++j) {
      const int64_t seen = len_k - len_q + j + 1;
      const int64_t t = cu_q[i] + j;
      ks[t] = cu_c[i];
      ke[t] = (int32_t)(cu_c[i] + std::min(seen / ratio, len_c));
    }
  }
}

}  // extern "C"
