/*
 * CSA2 CPU oracle.  TEST INFRASTRUCTURE ONLY: nothing on the product path may load,
 * link or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.
 *
 * A plain, slow, obviously correct host implementation of the CSA2 decode / chunked
 * prefill step: codecs -> indexer score -> Top-K -> gather + dequantise -> sparse softmax
 * attention -> layer modes.  Arithmetic is fp64 on the exact decoded values, except
 * where a step is defined by an fp32 operation whose result is a byte (the quantiser's
 * x / s and its scale, the coarse-key block mean): there the fp32 operation IS the
 * definition, so both implementations take the same integer decision.
 *
 * Sources (titles of the pages; section names as printed there):
 *   [N] "Detailed Notes On DeepSeek V4 Point 1 Flash In Simple Words":
 *       "Compressed Sparse Attention 2 Or CSA2 In Simple Terms",
 *       "The Three Modes Full Reindex And Reuse", "Hierarchical Sparse Indexer In Simple
 *       Terms", "FP4 Main KV Cache To Halve Storage Again", "Model Setup Numbers Without
 *       Jargon".
 *   [T] "DeepSeek-V4.1-Flash 技术解读" (mengman.github.io): 3.3 CSA2 (mode table and the
 *       figure caption on what each mode borrows), 3.4 Hierarchical Sparse Indexer,
 *       3.5 FP4 Main KV Cache.
 * Readings where the pages are silent are listed beside each function.
 *
 * Parallelism: OpenMP over independent (sequence, query) rows or cache rows only; every
 * output element is computed by one thread in one fixed order, so results do not depend
 * on the thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* Number formats                                                                        */
/* ------------------------------------------------------------------------------------ */

/* E2M1 (4 bits: sign, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 is
 * subnormal).  [N] "FP4 Main KV Cache", [T] 3.5: the main KV is stored as E2M1.
 * Value of the magnitude field m (0..7): e = m >> 1, f = m & 1;
 *   e == 0 : f * 0.5            (0, 0.5)
 *   e >= 1 : (1 + f/2) * 2^(e-1) (1, 1.5, 2, 3, 4, 6)                                   */
double orc_e2m1_value(int code) {
  int m = code & 7, e = m >> 1, f = m & 1;
  double mag = (e == 0) ? f * 0.5 : (1.0 + f * 0.5) * ldexp(1.0, e - 1);
  return (code & 8) ? -mag : mag;
}

/* Nearest E2M1 value to y, ties to the even code, saturating at +-6; the sign bit is the
 * sign of y even when the magnitude rounds to zero.  Brute force over the 8 magnitudes. */
int orc_e2m1_encode(float y) {
  double a = fabs((double)y);
  int best = 0;
  double best_d = INFINITY;
  for (int m = 0; m < 8; ++m) {
    double d = fabs(orc_e2m1_value(m) - a);
    if (d < best_d || (d == best_d && (m & 1) == 0 && (best & 1) == 1)) { best = m; best_d = d; }
  }
  if (isinf(y) || a > 6.0) best = 7;
  return best | (signbit(y) ? 8 : 0);
}

/* E4M3, OCP "FN" variant (8 bits: sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; exponent 15 with mantissa 7 is NaN; largest finite 448).
 *   e == 0 : m * 2^-9;   e >= 1 : (1 + m/8) * 2^(e-7).                                   */
double orc_e4m3_value(int code) {
  int e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return (code & 0x80) ? -mag : mag;
}

/* Nearest finite E4M3 value to y over the 127 magnitudes (codes 0x00..0x7E), ties to the
 * code with an even mantissa LSB, saturating at +-448, sign kept.  Brute force. */
int orc_e4m3_encode(float y) {
  double a = fabs((double)y);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 127; ++c) {
    double d = fabs(orc_e4m3_value(c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) { best = c; best_d = d; }
  }
  if (isinf(y) || a > 448.0) best = 126;
  return best | (signbit(y) ? 0x80 : 0);
}

/* ------------------------------------------------------------------------------------ */
/* Write side: quantise and pack                                                         */
/* ------------------------------------------------------------------------------------ */

/* FP4 main-KV quantisation with one fp32 scale per (sequence, channel).
 * [N] "FP4 Main KV Cache": entries are stored as E2M1 with a scale and decoded back
 * before attention.  The scale granularity here is one per channel over the whole
 * sequence (reading: the measured configurations state a per-channel absmax/6 scale;
 * the pages' own one-E4M3-scale-per-16-channels layout is a separate format).
 *   compute_scales = 1: s[b][c] = fl32(max_t |x[b][t][c]| / 6)      (build a cache)
 *   compute_scales = 0: s[b][c] is given (append rows to an existing cache)
 *   code = E2M1(fl32(x / s)); s == 0 gives code +0.
 * Row t of sequence b goes to cache row n0[b] + t (n0 == NULL: 0).  Two codes per byte,
 * the even channel in the low nibble.  x[b][t][c] is at x[b*xsb + t*xst + c].          */
void orc_quantize_fp4(int B, int T, int D, const float* x, int64_t xsb, int64_t xst, const int32_t* n0,
                      int64_t n_max, uint8_t* codes, float* scales, int compute_scales) {
  for (int b = 0; b < B; ++b) {
    float* s = scales + (int64_t)b * D;
    if (compute_scales) {
      for (int c = 0; c < D; ++c) {
        float amax = 0.0f;
        for (int t = 0; t < T; ++t) {
          float v = fabsf(x[b * xsb + t * xst + c]);
          if (v > amax) amax = v;
        }
        s[c] = amax / 6.0f;
      }
    }
    int64_t base = n0 ? n0[b] : 0;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
      uint8_t* row = codes + ((int64_t)b * n_max + base + t) * (D / 2);
      for (int c = 0; c < D; c += 2) {
        int lo = 0, hi = 0;
        if (s[c] != 0.0f) lo = orc_e2m1_encode(x[b * xsb + t * xst + c] / s[c]);
        if (s[c + 1] != 0.0f) hi = orc_e2m1_encode(x[b * xsb + t * xst + c + 1] / s[c + 1]);
        row[c / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* FP4 main-KV quantisation in the pages' own layout: E2M1 values with one E4M3 scale per
 * 16 consecutive channels of each entry and no second-level (global) scale.
 * [N] "FP4 Main KV Cache To Halve Storage Again" (one scale per 16 channels, no global
 * scale).  The pages do not say how the scale is chosen or rounded; reading (the plainest
 * one): the group's absmax divided by 6 (the largest E2M1 magnitude), rounded to E4M3 like
 * any other value (nearest, ties to even, saturating at 448), and the values divided by
 * that rounded scale:
 *   amax = max_{c in group} |x_c|;  sc = E4M3(fl32(amax / 6));  sv = value(sc)
 *   code_c = E2M1(fl32(x_c / sv)) (sv == 0 gives code +0)
 * A value can land above 6 after the division when the scale rounded down; E2M1 then
 * saturates it to 6.  codes [B][n_max][D/2] as in orc_quantize_fp4; gscales
 * [B][n_max][D/16] holds the E4M3 scale bytes.  D % 16 == 0. */
void orc_quantize_fp4_g16(int B, int T, int D, const float* x, int64_t xsb, int64_t xst, const int32_t* n0,
                          int64_t n_max, uint8_t* codes, uint8_t* gscales) {
  const int G = D / 16;
  for (int b = 0; b < B; ++b) {
    int64_t base = n0 ? n0[b] : 0;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
      const float* xr = x + b * xsb + t * xst;
      int64_t row = (int64_t)b * n_max + base + t;
      uint8_t* crow = codes + row * (D / 2);
      for (int g = 0; g < G; ++g) {
        float amax = 0.0f;
        for (int c = 16 * g; c < 16 * g + 16; ++c)
          if (fabsf(xr[c]) > amax) amax = fabsf(xr[c]);
        int sc = orc_e4m3_encode(amax / 6.0f);
        float sv = (float)orc_e4m3_value(sc);
        gscales[row * G + g] = (uint8_t)sc;
        for (int c = 16 * g; c < 16 * g + 16; c += 2) {
          int lo = 0, hi = 0;
          if (sv != 0.0f) {
            lo = orc_e2m1_encode(xr[c] / sv);
            hi = orc_e2m1_encode(xr[c + 1] / sv);
          }
          crow[c / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
  }
}

/* E4M3 quantisation with one fp32 scale per row (indexer keys, per token):
 *   s = fl32(max_d |x_d| / 448); code_d = E4M3(fl32(x_d / s)); s == 0 gives code +0.
 * Reading: the pages keep the indexer low-bit ([N] "FP4 Main KV Cache": indexer q/k
 * were already 4-bit in the previous model); the measured configurations store keys as
 * E4M3 with a per-token fp32 scale. */
void orc_quantize_fp8(int B, int T, int D, const float* x, int64_t xsb, int64_t xst, const int32_t* n0,
                      int64_t n_max, uint8_t* codes, float* scales) {
  for (int b = 0; b < B; ++b) {
    int64_t base = n0 ? n0[b] : 0;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
      const float* xr = x + b * xsb + t * xst;
      float amax = 0.0f;
      for (int d = 0; d < D; ++d)
        if (fabsf(xr[d]) > amax) amax = fabsf(xr[d]);
      float s = amax / 448.0f;
      int64_t row = (int64_t)b * n_max + base + t;
      scales[row] = s;
      for (int d = 0; d < D; ++d) codes[row * D + d] = (uint8_t)(s != 0.0f ? orc_e4m3_encode(xr[d] / s) : 0);
    }
  }
}

/* FP4 (E2M1) quantisation with one fp32 scale per row: the 4-bit indexer keys.
 * [N] "FP4 Main KV Cache To Halve Storage Again": the indexer queries and keys were already
 * 4-bit in the earlier model.  Reading (the pages give no layout): E2M1 with one fp32
 * scale per row, s = fl32(max_d |x_d| / 6), code = E2M1(fl32(x_d / s)) (s == 0 gives code
 * +0), two codes per byte with the even dim in the low nibble; codes [B][n_max][D/2],
 * scales [B][n_max]. */
void orc_quantize_fp4_rows(int B, int T, int D, const float* x, int64_t xsb, int64_t xst, const int32_t* n0,
                           int64_t n_max, uint8_t* codes, float* scales) {
  for (int b = 0; b < B; ++b) {
    int64_t base = n0 ? n0[b] : 0;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
      const float* xr = x + b * xsb + t * xst;
      float amax = 0.0f;
      for (int d = 0; d < D; ++d)
        if (fabsf(xr[d]) > amax) amax = fabsf(xr[d]);
      float s = amax / 6.0f;
      int64_t row = (int64_t)b * n_max + base + t;
      scales[row] = s;
      for (int d = 0; d < D; d += 2) {
        int lo = s != 0.0f ? orc_e2m1_encode(xr[d] / s) : 0;
        int hi = s != 0.0f ? orc_e2m1_encode(xr[d + 1] / s) : 0;
        codes[row * (D / 2) + d / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* Main-KV formats: 0 = one fp32 scale per (sequence, channel), scales [B][D];
 *                  2 = one E4M3 scale per 16 channels of each entry, scales [B][n_max][D/16]. */
enum { ORC_FMT_FP4_PER_CHANNEL = 0, ORC_FMT_FP4_G16 = 2 };

/* Dequantised value of channel c of FP4 cache row j of sequence b:
 *   per channel: fl32(E2M1(code) * s[b][c]);
 *   per 16 channels: E2M1(code) * E4M3(gs[b][j][c / 16]) (exact in fp32). */
static float fp4_dequant(int fmt, const uint8_t* codes, const void* scales, int b, int64_t n_max, int64_t j, int D,
                         int c) {
  const uint8_t* row = codes + ((int64_t)b * n_max + j) * (D / 2);
  int code = (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 15);
  double s;
  if (fmt == ORC_FMT_FP4_G16)
    s = orc_e4m3_value(((const uint8_t*)scales)[((int64_t)b * n_max + j) * (D / 16) + c / 16]);
  else
    s = ((const float*)scales)[(int64_t)b * D + c];
  return (float)(orc_e2m1_value(code) * s);
}

/* Gather + dequantise: out[b][t][k][c] = dequantised channel c of cache row idx[b][t][k];
 * rows with idx outside [0, n_max) (including the -1 padding) give 0. */
void orc_gather_dequant(int fmt, int B, int T, int K, int D, const uint8_t* codes, const void* scales, int64_t n_max,
                        const int32_t* idx, float* out) {
  for (int64_t r = 0; r < (int64_t)B * T * K; ++r) {
    int b = (int)(r / ((int64_t)T * K));
    int32_t j = idx[r];
    for (int c = 0; c < D; ++c)
      out[r * D + c] = (j >= 0 && j < n_max) ? fp4_dequant(fmt, codes, scales, b, n_max, j, D, c) : 0.0f;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Indexer                                                                               */
/* ------------------------------------------------------------------------------------ */

/* Indexer score of one query row against one key.  [N] "CSA2 In Simple Terms": each
 * layer's indexer (32 query heads, "Model Setup Numbers") scores the past entries.
 * The pages give no formula; reading: a head-weighted sum of per-head dot products,
 *     score_j = sum_h w_h * (q_h . k_j),
 * with no nonlinearity.
 *   prec 0 (fp32): q, k, w as given.
 *   prec 1 (fp8): the query is quantised per (token, head) to E4M3 with its own absmax/448
 *     scale sq_h (part of the definition; the pages keep indexer q and k low-bit), so
 *     score_j = sk_j * sum_h w_h * sq_h * sum_d E4M3(q8_hd) * E4M3(k8_jd).
 *   prec 2 (fp4): the same with E2M1 in place of E4M3 on both sides: the query quantised
 *     per (token, head) with sq_h = absmax/6, the keys from orc_quantize_fp4_rows.
 * q8 / sq are the pre-quantised query (prec 1, 2) or NULL; qf the fp32 query (prec 0). */
static double score_one(int prec, int H, int dk, const float* qf, const uint8_t* q8, const float* sq,
                        const float* w, const void* k, const float* k_scale, int64_t row) {
  double total = 0.0;
  if (prec == 0) {
    const float* kr = (const float*)k + row * dk;
    for (int h = 0; h < H; ++h) {
      double dot = 0.0;
      for (int d = 0; d < dk; ++d) dot += (double)qf[h * dk + d] * (double)kr[d];
      total += (double)w[h] * dot;
    }
  } else if (prec == 1) {
    const uint8_t* kr = (const uint8_t*)k + row * dk;
    for (int h = 0; h < H; ++h) {
      double dot = 0.0;
      for (int d = 0; d < dk; ++d) dot += orc_e4m3_value(q8[h * dk + d]) * orc_e4m3_value(kr[d]);
      total += (double)w[h] * (double)sq[h] * dot;
    }
    total *= (double)k_scale[row];
  } else {
    /* prec 2: E2M1 query codes (one per byte here) against packed E2M1 key codes */
    const uint8_t* kr = (const uint8_t*)k + row * (dk / 2);
    for (int h = 0; h < H; ++h) {
      double dot = 0.0;
      for (int d = 0; d < dk; ++d) {
        int kc = (d & 1) ? (kr[d / 2] >> 4) : (kr[d / 2] & 15);
        dot += orc_e2m1_value(q8[h * dk + d]) * orc_e2m1_value(kc);
      }
      total += (double)w[h] * (double)sq[h] * dot;
    }
    total *= (double)k_scale[row];
  }
  return total;
}

/* Per-(token, head) E2M1 quantisation of the indexer query (prec 2): sq = fl32(absmax/6),
 * code = E2M1(fl32(q / sq)), one code per byte. */
static void quantize_index_query_fp4(int rows, int dk, const float* q, uint8_t* q4, float* sq) {
  for (int r = 0; r < rows; ++r) {
    const float* qr = q + (int64_t)r * dk;
    float amax = 0.0f;
    for (int d = 0; d < dk; ++d)
      if (fabsf(qr[d]) > amax) amax = fabsf(qr[d]);
    float s = amax / 6.0f;
    sq[r] = s;
    for (int d = 0; d < dk; ++d) q4[(int64_t)r * dk + d] = (uint8_t)(s != 0.0f ? orc_e2m1_encode(qr[d] / s) : 0);
  }
}

/* Per-(token, head) E4M3 quantisation of the indexer query (prec 1). */
void orc_quantize_index_query(int rows, int dk, const float* q, uint8_t* q8, float* sq) {
  orc_quantize_fp8(1, rows, dk, q, 0, dk, NULL, rows, q8, sq);
}

/* Scores of B x T query rows.
 *   cand == NULL: column j is cache row j, j in [0, n_max); visible iff j < n_keys[b]
 *                 and (q_limit == NULL or j <= q_limit[b][t]).
 *   cand != NULL: column c is cache position cand[b][t][c]; visible iff that position is
 *                 >= 0 and passes the same tests.
 * Invisible columns get -inf.  scores is [B][T][ncols], ncols = cand ? C : n_max. */
void orc_index_score(int prec, int B, int T, int H, int dk, const float* q, const float* w, const void* k,
                     const float* k_scale, int64_t n_max, const int32_t* n_keys, const int32_t* q_limit,
                     const int32_t* cand, int C, double* scores) {
  int64_t ncols = cand ? C : n_max;
  uint8_t* q8 = (uint8_t*)malloc((size_t)B * T * H * dk + 1);
  float* sq = (float*)malloc(sizeof(float) * ((size_t)B * T * H + 1));
  if (prec == 1) orc_quantize_index_query(B * T * H, dk, q, q8, sq);
  if (prec == 2) quantize_index_query_fp4(B * T * H, dk, q, q8, sq);
  for (int64_t r = 0; r < (int64_t)B * T; ++r) {
    int b = (int)(r / T);
    int64_t limit = n_keys[b] - 1;
    if (limit > n_max - 1) limit = n_max - 1;
    if (q_limit && q_limit[r] < limit) limit = q_limit[r];
    const float* qf = q + r * H * dk;
    const uint8_t* qr8 = q8 + r * H * dk;
    const float* sqr = sq + r * H;
    const float* wr = w + r * H;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < ncols; ++c) {
      int64_t j = cand ? cand[r * C + c] : c;
      double v = -INFINITY;
      if (j >= 0 && j <= limit) v = score_one(prec, H, dk, qf, qr8, sqr, wr, k, k_scale, (int64_t)b * n_max + j);
      scores[r * ncols + c] = v;
    }
  }
  free(q8);
  free(sq);
}

/* ------------------------------------------------------------------------------------ */
/* Top-K                                                                                 */
/* ------------------------------------------------------------------------------------ */

typedef struct {
  double s;
  int64_t pos;
} scored_t;

/* Strict total order: higher score first, then lower position first. */
static int by_score_desc_pos_asc(const void* a, const void* b) {
  const scored_t* x = (const scored_t*)a;
  const scored_t* y = (const scored_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

static int by_pos_asc(const void* a, const void* b) {
  int64_t x = ((const scored_t*)a)->pos, y = ((const scored_t*)b)->pos;
  return (x < y) ? -1 : (x > y);
}

/* Top-K per row.  [N] "CSA2 In Simple Terms": the indexer keeps the 512 highest-scoring
 * past entries.  Reading (pages silent): ties go to the lower position; the result is
 * written in ascending position order and padded with -1 when fewer than K columns are
 * visible.  A column is visible iff its score is > -inf (NaN is not visible) and, with a
 * candidate list, its position is >= 0.  val_out (nullable) receives the selected
 * scores in the same order (-inf for padding). */
void orc_topk(int B, int T, int64_t ncols, const double* scores, const int32_t* cand, int K, int32_t* idx_out,
              double* val_out) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < (int64_t)B * T; ++r) {
    scored_t* v = (scored_t*)malloc(sizeof(scored_t) * (size_t)(ncols + 1));
    int64_t n = 0;
    for (int64_t c = 0; c < ncols; ++c) {
      double s = scores[r * ncols + c];
      int64_t pos = cand ? cand[r * ncols + c] : c;
      if (s > -INFINITY && pos >= 0) { v[n].s = s; v[n].pos = pos; ++n; }
    }
    qsort(v, (size_t)n, sizeof(scored_t), by_score_desc_pos_asc);
    int64_t keep = n < K ? n : K;
    qsort(v, (size_t)keep, sizeof(scored_t), by_pos_asc);
    for (int k = 0; k < K; ++k) {
      idx_out[r * K + k] = k < keep ? (int32_t)v[k].pos : -1;
      if (val_out) val_out[r * K + k] = k < keep ? v[k].s : -INFINITY;
    }
    free(v);
  }
}

/* ------------------------------------------------------------------------------------ */
/* Sparse attention                                                                      */
/* ------------------------------------------------------------------------------------ */

/* Softmax attention of each query row over only its selected entries.
 * [N] "CSA2 In Simple Terms" (attend to the selected top entries), "FP4 Main KV Cache"
 * (the FP4 codes become real values again only for attention), "Model Setup Numbers" (64 heads of
 * dim 512).  Reading: the whole dequantised entry is both key and value (K = V), so with
 * v_j the dequantised row j and S the selected rows (positions outside [0, n_max)
 * skipped):
 *   l_hj = scale * q_h . v_j;  m_h = max_j l_hj;  Z_h = sum_j exp(l_hj - m_h)
 *   o_h  = sum_j exp(l_hj - m_h) v_j / Z_h;   lse_h = m_h + ln Z_h
 * An empty S gives o = 0, lse = -inf.  q is [B][T][Hq][D]; out [B][T][Hq][D]; lse
 * [B][T][Hq] (nullable); fmt and scales as for fp4_dequant.
 * Sliding window (swa_codes != NULL): [N] "CSA2 In Simple Terms" (every layer also looks
 * at recent tokens through sliding window attention), "Model Setup Numbers" (window 128),
 * "FP4 Main KV Cache" (the window cache stays 8-bit), 3.3 of the Chinese reading (each
 * layer keeps its own window KV).  Reading: the window's entries join S in one softmax
 * (the whole entry again both key and value); the window cache is E4M3 with one fp32
 * scale per row (swa_codes [B][swa_n_max][D], swa_scales [B][swa_n_max]); row (b,t)
 * sees window rows [max(0, e - window), e) with e = min(swa_end[b][t], swa_n_max). */
void orc_sparse_attend(int fmt, int B, int T, int Hq, int D, const float* q, const uint8_t* codes,
                       const void* scales, int64_t n_max, const int32_t* idx, int K, const uint8_t* swa_codes,
                       const float* swa_scales, int64_t swa_n_max, const int32_t* swa_end, int window,
                       double scale, double* out, double* lse) {
  const int W = swa_codes ? window : 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < (int64_t)B * T; ++r) {
    int b = (int)(r / T);
    double* v = (double*)malloc(sizeof(double) * (size_t)(K + W) * D);
    double* l = (double*)malloc(sizeof(double) * (size_t)(K + W));
    int n = 0;
    for (int k = 0; k < K; ++k) {
      int32_t j = idx[r * K + k];
      if (j < 0 || j >= n_max) continue;
      for (int c = 0; c < D; ++c) v[(int64_t)n * D + c] = fp4_dequant(fmt, codes, scales, b, n_max, j, D, c);
      ++n;
    }
    /* the sliding window: the last `window` entries before swa_end[b][t] of this layer's
     * own cache, dequantised as E4M3(code) * s_row, joining the same softmax */
    if (W > 0) {
      int64_t end = swa_end[r];
      if (end > swa_n_max) end = swa_n_max;
      int64_t start = end - W < 0 ? 0 : end - W;
      for (int64_t j = start; j < end; ++j) {
        const int64_t row = (int64_t)b * swa_n_max + j;
        for (int c = 0; c < D; ++c)
          v[(int64_t)n * D + c] = orc_e4m3_value(swa_codes[row * D + c]) * (double)swa_scales[row];
        ++n;
      }
    }
    for (int h = 0; h < Hq; ++h) {
      const float* qh = q + (r * Hq + h) * D;
      double* oh = out + (r * Hq + h) * D;
      for (int c = 0; c < D; ++c) oh[c] = 0.0;
      if (n == 0) {
        if (lse) lse[r * Hq + h] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (int i = 0; i < n; ++i) {
        double dot = 0.0;
        for (int c = 0; c < D; ++c) dot += (double)qh[c] * v[(int64_t)i * D + c];
        l[i] = scale * dot;
        if (l[i] > m) m = l[i];
      }
      double z = 0.0;
      for (int i = 0; i < n; ++i) {
        double p = exp(l[i] - m);
        z += p;
        for (int c = 0; c < D; ++c) oh[c] += p * v[(int64_t)i * D + c];
      }
      for (int c = 0; c < D; ++c) oh[c] /= z;
      if (lse) lse[r * Hq + h] = m + log(z);
    }
    free(v);
    free(l);
  }
}

/* ------------------------------------------------------------------------------------ */
/* Two-level indexer: coarse keys                                                        */
/* ------------------------------------------------------------------------------------ */

/* Coarse indexer keys: for each block of `block` consecutive cache rows, the mean of the
 * dequantised E4M3 keys, re-quantised to E4M3 with its own absmax/448 scale.
 * Reading (the pages' hierarchical indexer ranks blocks of positions; the measured
 * long-context configuration ranks blocks by a mean key): the mean is defined in fp32,
 *   mean_c = fl32( (sum over j in block, in j order, of fl32(sk_j * E4M3(k8_jc))) / count )
 * with each partial sum rounded to fp32, so that the re-quantised bytes are reproducible.
 * Blocks cover [0, n_keys[b]); the last block may be partial; blocks at or past
 * ceil(n_keys/block) are zero with scale 0.  kb8 is [B][nb_max][dk], kb_scale [B][nb_max],
 * nb_max = ceil(n_max / block). */
void orc_coarse_keys(int B, int64_t n_max, const int32_t* n_keys, int dk, int block, const uint8_t* k8,
                     const float* k_scale, uint8_t* kb8, float* kb_scale) {
  int64_t nb_max = (n_max + block - 1) / block;
  for (int b = 0; b < B; ++b) {
    int64_t nk = n_keys[b] < n_max ? n_keys[b] : n_max;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < nb_max; ++blk) {
      float mean[1024];
      int64_t j0 = blk * block, j1 = j0 + block < nk ? j0 + block : nk;
      int64_t out_row = (int64_t)b * nb_max + blk;
      if (j1 <= j0) {
        kb_scale[out_row] = 0.0f;
        memset(kb8 + out_row * dk, 0, (size_t)dk);
        continue;
      }
      for (int c = 0; c < dk; ++c) {
        float sum = 0.0f;
        for (int64_t j = j0; j < j1; ++j) {
          int64_t row = (int64_t)b * n_max + j;
          float v = (float)(orc_e4m3_value(k8[row * dk + c]) * (double)k_scale[row]);
          sum = sum + v;
        }
        mean[c] = sum / (float)(j1 - j0);
      }
      orc_quantize_fp8(1, 1, dk, mean, 0, 0, NULL, 1, kb8 + out_row * dk, kb_scale + out_row);
    }
  }
}

/* Threads the oracle's parallel loops use (for reporting the CPU baseline). */
int orc_num_threads(void) { return omp_get_max_threads(); }
