/*
 * pda_oracle.c -- fp64 CPU oracle for single-token decode attention over a
 * paged KV cache.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the benchmark's CPU-baseline leg call it; the product path never does.
 * It shares no code, header or constant with the HIP path.
 *
 * What it computes is the plain definition, written out with no blocking,
 * fusion or reordering (each step cites the page it follows):
 *
 *   for every sequence b and query head h:
 *     kvh  = floor(h / G), G = Hq / Hkv           (contiguous grouping:
 *            "From MHA to MLA", sec. 2, the GQA kernel's kv_head line, and
 *            the drill page, sec. 8, first pitfall)
 *     gather, for logical token j < n_b:
 *            page = block_tables[b][floor(j / P)], slot = j mod P
 *            K_j = dec(k_cache[page, slot, kvh, :]) * k_scale
 *            V_j = dec(v_cache[page, slot, kvh, :]) * v_scale
 *            (paged addressing: "From MHA to MLA", sec. 5; drill page, sec. 4)
 *     s_j  = scale * sum_i q_i K_j,i
 *     m    = max_j s_j ; Z = sum_j exp(s_j - m)
 *     out  = sum_j exp(s_j - m) V_j / Z ;  lse = m + ln Z
 *            (softmax and natural-log LSE of the scaled logits: "From MHA to
 *            MLA", sec. 2 kernel epilogue; FlashMLA-ETAP "Usage", lse)
 *
 *   MLA ("From MHA to MLA", sec. 6; "Attention Kernel Variants", MLA section):
 *     one cache record per token [c (d_latent) | k_R (d_rope)], no head axis.
 *     K_j = the whole record, V_j = its first d_latent values (same bytes),
 *     s_j = scale * (q[:d_latent] . c_j + q[d_latent:] . k_R_j).
 *
 *   Several query tokens per sequence (multi-token decode: FlashMLA-ETAP
 *   "Supported configurations", query length, and "Usage", the q / o / lse
 *   shapes): q [B, s_q, Hq, d], out [B, s_q, Hq, dv], lse [B, Hq, s_q].  With
 *   the causal mask aligned bottom-right ("From MHA to MLA", sec. 2, the
 *   reference kernel's causal branch) query i of s_q sits at position
 *   n - s_q + i and sees keys j <= that position, i.e. the first
 *   n - (s_q - 1 - i) tokens; without the mask every query sees all n.  A
 *   query that sees no token is empty (out = 0, lse = -inf).  s_q = 1 is
 *   the single-token case above, where the mask removes nothing.
 *
 *   Split-KV (Flash-Decoding, "From MHA to MLA", sec. 4): attention over a
 *   token interval gives a normalized partial O_s and L_s; the combine is
 *     L = ln sum_s exp(L_s),  O = sum_s exp(L_s - L) O_s,
 *   evaluated with the maximum L_s subtracted first.  Empty intervals give
 *   O_s = 0, L_s = -inf and weight 0.
 *
 * Element decoders are written from the format definitions (IEEE binary16,
 * bfloat16 = the top half of binary32, OCP FP8 E4M3FN: bias 7, no infinities,
 * S.1111.111 is NaN).
 *
 * Every table entry the oracle dereferences is bounds-checked against the
 * pool: an out-of-range entry returns ORC_ERR_TABLE instead of reading.
 *
 * Parity pins live in tests/test_oracle_*.py (brute force, library SDPA,
 * closed forms, invariants, the pages' printed numbers).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3, ORC_F64 = 4 };
enum { ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_TABLE = 2, ORC_ERR_NOMEM = 3 };

/* ---------------------------------------------------------------- decoders */

static double dec_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-10 * 2^-14 */
  } else if (e == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  }
  return sign ? -v : v;
}

static double dec_bf16(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xff;
  int m = b & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -133); /* subnormal: m * 2^-7 * 2^-126 */
  } else if (e == 255) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp(1.0 + (double)m / 128.0, e - 127);
  }
  return sign ? -v : v;
}

static double dec_e4m3(uint8_t x) {
  int sign = (x >> 7) & 1;
  int e = (x >> 3) & 0xf;
  int m = x & 0x7;
  double v;
  if (e == 15 && m == 7) {
    v = NAN; /* the only NaN encodings of E4M3FN; there is no infinity */
  } else if (e == 0) {
    v = ldexp((double)m, -9); /* subnormal: m * 2^-3 * 2^-6 */
  } else {
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  }
  return sign ? -v : v;
}

static double dec_elem(int dtype, const void* base, int64_t i) {
  switch (dtype) {
    case ORC_F32: {
      float f;
      memcpy(&f, (const char*)base + 4 * i, 4);
      return (double)f;
    }
    case ORC_F16: {
      uint16_t h;
      memcpy(&h, (const char*)base + 2 * i, 2);
      return dec_f16(h);
    }
    case ORC_BF16: {
      uint16_t b;
      memcpy(&b, (const char*)base + 2 * i, 2);
      return dec_bf16(b);
    }
    case ORC_E4M3:
      return dec_e4m3(((const uint8_t*)base)[i]);
    case ORC_F64: {
      double d;
      memcpy(&d, (const char*)base + 8 * i, 8);
      return d;
    }
  }
  return NAN;
}

/* Decode n elements of one dtype starting at element index i0 (exported so
 * the tests can pin the decoders against library dtype casts). */
int orc_decode(int dtype, const void* base, int64_t i0, int64_t n, double* out) {
  if (dtype < ORC_F32 || dtype > ORC_F64 || !base || !out || n < 0) return ORC_ERR_ARG;
  for (int64_t k = 0; k < n; ++k) out[k] = dec_elem(dtype, base, i0 + k);
  return ORC_OK;
}

/* ------------------------------------------------------- one head, fp64 */

/* Softmax attention of one query row over n contiguous gathered rows.
 * K is [n][dk], V is [n][dv] (fp64).  Two passes: max, then sums. */
static void attend_rows(const double* q, const double* K, const double* V, int64_t n,
                        int dk, int dv, double scale, double* s, double* out,
                        double* lse) {
  for (int e = 0; e < dv; ++e) out[e] = 0.0;
  if (n == 0) { /* defensive definition for an empty interval */
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += q[i] * K[j * dk + i];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    double w = exp(s[j] - m);
    z += w;
    for (int e = 0; e < dv; ++e) out[e] += w * V[j * dv + e];
  }
  for (int e = 0; e < dv; ++e) out[e] /= z;
  *lse = m + log(z);
}

/* Gather tokens [t0, t1) of sequence b for one cache head into contiguous
 * fp64 rows.  rec_stride: elements between consecutive tokens in a page;
 * page_stride: elements between pages; off: element offset of the head's
 * row inside a token record; width: how many elements to take. */
static int gather_rows(const void* cache, int dtype, const int32_t* table_row,
                       int64_t num_pages, int P, int64_t page_stride,
                       int64_t rec_stride, int64_t off, int width, double mult,
                       int64_t t0, int64_t t1, double* dst) {
  for (int64_t j = t0; j < t1; ++j) {
    int32_t page = table_row[j / P];
    if (page < 0 || (int64_t)page >= num_pages) return ORC_ERR_TABLE;
    int64_t slot = j % P;
    int64_t base = (int64_t)page * page_stride + slot * rec_stride + off;
    for (int i = 0; i < width; ++i)
      dst[(j - t0) * width + i] = dec_elem(dtype, cache, base + i) * mult;
  }
  return ORC_OK;
}

/* Tokens query i of q_len may see in a sequence of n cached tokens. */
static int64_t visible_tokens(int64_t n, int q_len, int i, int causal) {
  int64_t v = causal ? n - (int64_t)(q_len - 1 - i) : n;
  return v > 0 ? v : 0;
}

/* ------------------------------------------------------------- GQA / MHA */

/* Paged decode attention, GQA family.
 *   q            [B, q_len, Hq, dk] of q_dtype
 *   k_cache      [num_pages, P, Hkv, dk] of kv_dtype
 *   v_cache      [num_pages, P, Hkv, dv] of kv_dtype
 *   block_tables [B, max_pages] int32, context_lens [B] int32
 *   tok_begin/tok_end [B] int32 or NULL: restrict to tokens [begin, end)
 *     of each sequence (a split interval); NULL means [0, n_b).  A query
 *     takes the part of that interval it may see (causal: see the header).
 *   row_mask [B*q_len*Hq] or NULL: compute only rows with a nonzero mask.
 *   out [B, q_len, Hq, dv] fp64, lse [B, Hq, q_len] fp64 (rows not computed
 *   are untouched).
 * Returns ORC_OK, ORC_ERR_ARG or ORC_ERR_TABLE.  num_threads <= 0: default. */
int orc_paged_attention(const void* q, int q_dtype, const void* k_cache,
                        const void* v_cache, int kv_dtype,
                        const int32_t* block_tables, int max_pages,
                        const int32_t* context_lens, const int32_t* tok_begin,
                        const int32_t* tok_end, int B, int q_len, int Hq, int Hkv,
                        int dk, int dv, int P, int64_t num_pages, double scale,
                        double k_scale, double v_scale, int causal,
                        const uint8_t* row_mask, double* out, double* lse,
                        int num_threads) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !lse)
    return ORC_ERR_ARG;
  if (B < 0 || q_len <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || dk <= 0 || dv <= 0 ||
      P <= 0 || max_pages < 0 || num_pages < 0)
    return ORC_ERR_ARG;
  const int G = Hq / Hkv;
  int status = ORC_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < (int64_t)B * q_len * Hq; ++r) {
    if (row_mask && !row_mask[r]) continue;
    /* row r = (b, query i, head h) of out [B, q_len, Hq, dv] */
    int b = (int)(r / ((int64_t)q_len * Hq));
    int i = (int)((r / Hq) % q_len);
    int h = (int)(r % Hq);
    int kvh = h / G;
    int64_t lse_row = ((int64_t)b * Hq + h) * q_len + i;
    int64_t n_b = context_lens[b];
    int64_t t0 = tok_begin ? tok_begin[b] : 0;
    int64_t t1 = tok_end ? tok_end[b] : n_b;
    if (n_b < 0 || t0 < 0 || t1 > n_b || t1 > (int64_t)max_pages * P) {
#pragma omp atomic write
      status = ORC_ERR_ARG;
      continue;
    }
    int64_t vis = visible_tokens(n_b, q_len, i, causal);
    if (t1 > vis) t1 = vis;
    if (t1 < t0) t1 = t0;
    int64_t n = t1 - t0;
    double* qd = (double*)malloc(sizeof(double) * dk);
    double* K = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * dk);
    double* V = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * dv);
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!qd || !K || !V || !s) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    } else {
      for (int e = 0; e < dk; ++e) qd[e] = dec_elem(q_dtype, q, r * dk + e);
      const int32_t* trow = block_tables + (int64_t)b * max_pages;
      int rk = gather_rows(k_cache, kv_dtype, trow, num_pages, P, (int64_t)P * Hkv * dk,
                           (int64_t)Hkv * dk, (int64_t)kvh * dk, dk, k_scale, t0, t1, K);
      int rv = gather_rows(v_cache, kv_dtype, trow, num_pages, P, (int64_t)P * Hkv * dv,
                           (int64_t)Hkv * dv, (int64_t)kvh * dv, dv, v_scale, t0, t1, V);
      if (rk != ORC_OK || rv != ORC_OK) {
#pragma omp atomic write
        status = ORC_ERR_TABLE;
      } else {
        attend_rows(qd, K, V, n, dk, dv, scale, s, out + r * dv, lse + lse_row);
      }
    }
    free(qd);
    free(K);
    free(V);
    free(s);
  }
  return status;
}

/* ------------------------------------------------------------------- MLA */

/* Paged decode attention over an MLA latent cache (one record per token, no
 * head axis).  q [B, q_len, Hq, d_latent + d_rope]; kv_cache [num_pages, P,
 * d_latent + d_rope]; out [B, q_len, Hq, d_latent] fp64; lse [B, Hq, q_len]
 * fp64.  K_j is the whole record times kv_scale (the dequantization scale of
 * an fp8 latent, 1 otherwise), V_j its first d_latent values (the same
 * scaled values); queries and the causal mask as in orc_paged_attention. */
int orc_mla_attention(const void* q, int q_dtype, const void* kv_cache, int kv_dtype,
                      const int32_t* block_tables, int max_pages,
                      const int32_t* context_lens, const int32_t* tok_begin,
                      const int32_t* tok_end, int B, int q_len, int Hq, int d_latent,
                      int d_rope, int P, int64_t num_pages, double scale, double kv_scale,
                      int causal, const uint8_t* row_mask, double* out, double* lse,
                      int num_threads) {
  if (!q || !kv_cache || !block_tables || !context_lens || !out || !lse) return ORC_ERR_ARG;
  if (B < 0 || q_len <= 0 || Hq <= 0 || d_latent <= 0 || d_rope < 0 || P <= 0 ||
      max_pages < 0 || num_pages < 0)
    return ORC_ERR_ARG;
  const int rec = d_latent + d_rope;
  int status = ORC_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < (int64_t)B * q_len * Hq; ++r) {
    if (row_mask && !row_mask[r]) continue;
    int b = (int)(r / ((int64_t)q_len * Hq));
    int i = (int)((r / Hq) % q_len);
    int h = (int)(r % Hq);
    int64_t lse_row = ((int64_t)b * Hq + h) * q_len + i;
    int64_t n_b = context_lens[b];
    int64_t t0 = tok_begin ? tok_begin[b] : 0;
    int64_t t1 = tok_end ? tok_end[b] : n_b;
    if (n_b < 0 || t0 < 0 || t1 > n_b || t1 > (int64_t)max_pages * P) {
#pragma omp atomic write
      status = ORC_ERR_ARG;
      continue;
    }
    int64_t vis = visible_tokens(n_b, q_len, i, causal);
    if (t1 > vis) t1 = vis;
    if (t1 < t0) t1 = t0;
    int64_t n = t1 - t0;
    double* qd = (double*)malloc(sizeof(double) * rec);
    double* K = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * rec);
    double* V = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * d_latent);
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!qd || !K || !V || !s) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    } else {
      for (int e = 0; e < rec; ++e) qd[e] = dec_elem(q_dtype, q, r * rec + e);
      const int32_t* trow = block_tables + (int64_t)b * max_pages;
      /* K: the whole record; V: the latent part of the same record. */
      int rk = gather_rows(kv_cache, kv_dtype, trow, num_pages, P, (int64_t)P * rec, rec, 0,
                           rec, kv_scale, t0, t1, K);
      int rv = gather_rows(kv_cache, kv_dtype, trow, num_pages, P, (int64_t)P * rec, rec, 0,
                           d_latent, kv_scale, t0, t1, V);
      if (rk != ORC_OK || rv != ORC_OK) {
#pragma omp atomic write
        status = ORC_ERR_TABLE;
      } else {
        attend_rows(qd, K, V, n, rec, d_latent, scale, s, out + r * d_latent, lse + lse_row);
      }
    }
    free(qd);
    free(K);
    free(V);
    free(s);
  }
  return status;
}

/* ------------------------------------------------------------- KV append */

static size_t elem_size(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_E4M3: return 1;
    case ORC_F64: return 8;
    default: return 0;
  }
}

/* The E4M3FN byte nearest to x (already a float value), by search over every
 * finite code: ties go to the code with an even mantissa; magnitudes beyond
 * 448, infinities included, saturate to 448; NaN gives 0x7F. */
static uint8_t enc_e4m3(double x) {
  if (x != x) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a > 448.0) a = 448.0;
  uint8_t best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(dec_e4m3((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = (uint8_t)c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* Write s_new new tokens per sequence into one paged cache tensor (the blog,
 * sec. 2: the new token's key and value join the cache before attention;
 * sec. 5 and the drill page sec. 4: block-table addressing).
 *   src   [B, s_new, H, width] of src_dtype
 *   cache [num_pages, P, H, width] of cache_dtype
 *   token t of sequence b, at position p = positions[b] + t, goes to
 *   cache[block_tables[b][p / P], p % P, :, :]; positions[b] < 0 skips b.
 * Same dtype: the elements are copied.  E4M3 cache (src f32/f16/bf16): the
 * byte is the E4M3FN value nearest to the fp32 quotient x / scale, ties to
 * even, saturated at +-448.  Other pairs: ORC_ERR_ARG.  Every table entry
 * and position is bounds-checked (ORC_ERR_TABLE / ORC_ERR_ARG, nothing
 * written for that token). */
int orc_kv_append(const void* src, int src_dtype, void* cache, int cache_dtype,
                  const int32_t* block_tables, int max_pages, const int32_t* positions, int B,
                  int s_new, int H, int width, int P, int64_t num_pages, float scale) {
  if (!src || !cache || !block_tables || !positions || B < 0 || s_new < 0 || H <= 0 ||
      width <= 0 || P <= 0 || max_pages < 0 || num_pages < 0)
    return ORC_ERR_ARG;
  const int quant = cache_dtype == ORC_E4M3;
  if (quant ? !(src_dtype == ORC_F32 || src_dtype == ORC_F16 || src_dtype == ORC_BF16)
            : src_dtype != cache_dtype)
    return ORC_ERR_ARG;
  if (quant && !(scale > 0.0f)) return ORC_ERR_ARG;
  const size_t es = elem_size(cache_dtype);
  const int64_t row = (int64_t)H * width; /* elements of one token */
  int status = ORC_OK;
  for (int b = 0; b < B; ++b) {
    if (positions[b] < 0) continue;
    for (int t = 0; t < s_new; ++t) {
      int64_t p = (int64_t)positions[b] + t;
      if (p >= (int64_t)max_pages * P) {
        status = ORC_ERR_ARG;
        continue;
      }
      int32_t page = block_tables[(int64_t)b * max_pages + p / P];
      if (page < 0 || (int64_t)page >= num_pages) {
        status = ORC_ERR_TABLE;
        continue;
      }
      int64_t dst0 = ((int64_t)page * P + p % P) * row;
      int64_t src0 = ((int64_t)b * s_new + t) * row;
      for (int64_t i = 0; i < row; ++i) {
        if (quant) {
          float x = (float)dec_elem(src_dtype, src, src0 + i); /* exact: f32/f16/bf16 */
          float q = x / scale;                                 /* one fp32 division */
          ((uint8_t*)cache)[dst0 + i] = enc_e4m3((double)q);
        } else {
          memcpy((char*)cache + (dst0 + i) * es, (const char*)src + (src0 + i) * es, es);
        }
      }
    }
  }
  return status;
}

/* --------------------------------------------------------------- combine */

/* LSE-weighted merge of S split partials ("From MHA to MLA", sec. 4).
 *   part_o [R, S, dv] fp64, part_lse [R, S] fp64 -> out [R, dv], lse [R].
 * A split with part_lse = -inf is empty and gets weight 0; if every split is
 * empty the row is empty: out = 0, lse = -inf. */
int orc_combine(const double* part_o, const double* part_lse, int64_t R, int S, int dv,
                double* out, double* lse) {
  if (!part_o || !part_lse || !out || !lse || R < 0 || S <= 0 || dv <= 0) return ORC_ERR_ARG;
  for (int64_t r = 0; r < R; ++r) {
    double mx = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (part_lse[r * S + s] > mx) mx = part_lse[r * S + s];
    for (int e = 0; e < dv; ++e) out[r * dv + e] = 0.0;
    if (mx == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double denom = 0.0;
    for (int s = 0; s < S; ++s) {
      double l = part_lse[r * S + s];
      if (l == -INFINITY) continue;
      double w = exp(l - mx);
      denom += w;
      for (int e = 0; e < dv; ++e) out[r * dv + e] += w * part_o[(r * S + s) * dv + e];
    }
    for (int e = 0; e < dv; ++e) out[r * dv + e] /= denom;
    lse[r] = mx + log(denom);
  }
  return ORC_OK;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
