/*
 * oracle.c -- plain CPU oracle for index-selected sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
 * CPU-baseline leg are its only users. The GPU library never links, loads or
 * calls it, and the two share no code.
 *
 * What is computed follows three pages:
 *  [P1] "Day-0 Inference Adaptation for Ultra-Large MoE Models on Domestic GPUs:
 *       A Software Stack Perspective", sections "Adapting Sparse Attention:
 *       Indexing, Caching, and Dual-Path Execution", "Operatorizing Index
 *       Selection", "Reorganizing KV Cache Layout".
 *  [P2] "Day-0 Inference Adaptation of Ultra-Large-Scale MoE Models on Domestic
 *       AI Accelerators", section 4.1 "Sparse Attention Index Pipeline".
 *  [P3] "Day-0 Adaptation for Trillion-Parameter MoE Models: A Comprehensive
 *       Guide to Heterogeneous Compute Deployment", section IV "Sparse Attention
 *       Path: Index Selection, KV Layout, and Two-Phase Computation".
 *
 * The method: score compressed query/key representations, keep the top-k
 * positions per query, gather those rows from a block-organised KV cache and
 * run exact attention over them only [P2 4.1]. The variant of [P1
 * "Operatorizing Index Selection"] and [P2 4.1] first prunes whole blocks and
 * then selects exactly inside the surviving blocks.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - scores are a plain dot product with no scale and no nonlinearity;
 *  - the causal boundary is inclusive: query at p sees positions 0..p;
 *  - ties are broken by lower position (score descending, then position
 *    ascending); pages by lower logical page index; -0.0 equals +0.0;
 *  - fewer candidates than topk: all are taken, idx is padded with -1;
 *  - idx is returned in ascending position order and w holds the selected
 *    scores; w does not enter the attention, which is a plain softmax of the
 *    scaled q.k logits over the selected set;
 *  - the page maximum of the last, partial page runs over its valid positions.
 *
 * Precision: scores are summed in fp64 and rounded once to fp32, and the
 * selection runs on those fp32 values. Attention is computed in fp64.
 * Nothing here is blocked, fused or reordered: full sorts and dense loops.
 *
 * The second workload of the pages is the online conversion of low-precision
 * expert weights ([P1] "Handling Low-Precision Expert Weights: Online
 * Conversion and Workspace Reuse"; [P3] section V "Low-Bit Expert Weights:
 * Online Conversion and Workspace Reuse"): MXFP4 blocks are dequantised into
 * an FP8 working format just before use. Each element's exact value is
 * formed in fp64 from the format definitions and rounded once to E4M3.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int g_threads = 1;

int oracle_set_threads(int n) {
  if (n < 1) return -1;
  g_threads = n;
  return 0;
}

int oracle_get_threads(void) { return g_threads; }

/* bf16 bit pattern -> its exact value */
static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* fp32 -> bf16, round to nearest, ties to even */
static uint16_t fp32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
    return (uint16_t)((u >> 16) | 0x0040u); /* keep NaN a (quiet) NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* position of query row i of sequence b */
static int64_t query_position(const oracle_shape* sh, const int32_t* seq_lens,
                              const int32_t* q_start, int b, int i) {
  int64_t first = q_start ? (int64_t)q_start[b] : (int64_t)seq_lens[b] - sh->num_q;
  return first + i;
}

/* row of logical position j of sequence b in a paged cache [P][bs][...] */
static int64_t physical_row(const oracle_shape* sh, const int32_t* page_table, int b,
                            int64_t j) {
  int64_t page = page_table[(int64_t)b * sh->max_pages + j / sh->block_size];
  return page * sh->block_size + j % sh->block_size;
}

static int shape_ok(const oracle_shape* sh) {
  return sh && sh->batch > 0 && sh->num_q > 0 && sh->block_size > 0 && sh->max_pages > 0 &&
         sh->num_idx_heads >= 0;
}

/* indexer heads: every (query row, indexer head) is one selection row */
static int idx_heads(const oracle_shape* sh) {
  return sh->num_idx_heads > 1 ? sh->num_idx_heads : 1;
}

/* ---------------------------------------------------------------- scoring */

int oracle_index_scores(const oracle_shape* sh, const uint16_t* q_comp,
                        const uint16_t* k_comp_cache, const int32_t* page_table,
                        const int32_t* seq_lens, const int32_t* q_start,
                        float* scores, int64_t ld) {
  if (!shape_ok(sh) || sh->d_c <= 0 || !q_comp || !k_comp_cache || !page_table || !scores)
    return -1;
  if (!q_start && !seq_lens) return -1;
  const int hi = idx_heads(sh);
  const int64_t rows = (int64_t)sh->batch * sh->num_q * hi;
  const int64_t limit = (int64_t)sh->max_pages * sh->block_size;
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t qr = r / hi;
    int64_t p = query_position(sh, seq_lens, q_start, (int)(qr / sh->num_q), (int)(qr % sh->num_q));
    if (p >= limit || p >= ld) return -1;
  }
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
  for (int64_t r = 0; r < rows; ++r) {
    /* selection row r: query row r / hi, indexer head r % hi */
    const int64_t qr = r / hi;
    const int b = (int)(qr / sh->num_q), i = (int)(qr % sh->num_q);
    const int64_t p = query_position(sh, seq_lens, q_start, b, i);
    const uint16_t* qc = q_comp + r * sh->d_c;
    float* out = scores + r * ld;
    for (int64_t j = 0; j <= p; ++j) {
      const uint16_t* kc = k_comp_cache + physical_row(sh, page_table, b, j) * sh->d_c;
      double acc = 0.0;
      for (int c = 0; c < sh->d_c; ++c) acc += bf16_value(qc[c]) * bf16_value(kc[c]);
      out[j] = (float)acc;
    }
  }
  return 0;
}

/* -------------------------------------------------------------- selection */

typedef struct {
  float key;  /* score, or page maximum */
  int64_t at; /* position, or logical page */
} ranked;

/* larger key first; equal keys: lower index first */
static int higher_key_then_lower_index(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->key > b->key) return -1;
  if (a->key < b->key) return 1;
  return (a->at > b->at) - (a->at < b->at);
}

static int lower_index(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  return (a->at > b->at) - (a->at < b->at);
}

int oracle_topk_select(const oracle_shape* sh, const float* scores, int64_t ld,
                       const int32_t* seq_lens, const int32_t* q_start,
                       int32_t topk, int32_t n_sel_pages,
                       int32_t* idx, float* w, int32_t* count,
                       uint64_t* page_mask, int32_t* sel_pages) {
  if (!shape_ok(sh) || !scores || topk <= 0 || n_sel_pages < 0) return -1;
  if (!q_start && !seq_lens) return -1;
  const int hi = idx_heads(sh);
  const int64_t rows = (int64_t)sh->batch * sh->num_q * hi;
  const int64_t bs = sh->block_size;
  const int64_t limit = (int64_t)sh->max_pages * bs;
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t qr = r / hi;
    int64_t p = query_position(sh, seq_lens, q_start, (int)(qr / sh->num_q), (int)(qr % sh->num_q));
    if (p >= limit || p >= ld) return -1;
  }
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
  for (int64_t r = 0; r < rows; ++r) {
    /* selection row r: query row r / hi, indexer head r % hi */
    const int64_t qr = r / hi;
    const int b = (int)(qr / sh->num_q), i = (int)(qr % sh->num_q);
    const int64_t p = query_position(sh, seq_lens, q_start, b, i);
    const float* s = scores + r * ld;
    const int64_t n_valid = p >= 0 ? p + 1 : 0;

    /* the candidate set */
    ranked* cand = (ranked*)malloc(sizeof(ranked) * (size_t)(n_valid > 0 ? n_valid : 1));
    int64_t m = 0;
    int64_t n_pg = n_valid > 0 ? p / bs + 1 : 0;
    int64_t n_keep_pages = 0;
    ranked* pages = NULL;
    if (n_sel_pages == 0) {
      for (int64_t j = 0; j < n_valid; ++j) {
        cand[m].key = s[j];
        cand[m].at = j;
        ++m;
      }
    } else {
      /* block granularity first: the maximum score of each page over its
         valid positions, then the best n_sel_pages pages */
      pages = (ranked*)malloc(sizeof(ranked) * (size_t)(n_pg > 0 ? n_pg : 1));
      for (int64_t g = 0; g < n_pg; ++g) {
        int64_t last = g * bs + bs - 1 < p ? g * bs + bs - 1 : p;
        float mx = s[g * bs];
        for (int64_t j = g * bs + 1; j <= last; ++j)
          if (s[j] > mx) mx = s[j];
        pages[g].key = mx;
        pages[g].at = g;
      }
      qsort(pages, (size_t)n_pg, sizeof(ranked), higher_key_then_lower_index);
      n_keep_pages = n_pg < n_sel_pages ? n_pg : n_sel_pages;
      char* keep = (char*)calloc((size_t)(n_pg > 0 ? n_pg : 1), 1);
      for (int64_t t = 0; t < n_keep_pages; ++t) keep[pages[t].at] = 1;
      /* then exact selection among the tokens of the kept pages */
      for (int64_t j = 0; j < n_valid; ++j) {
        if (keep[j / bs]) {
          cand[m].key = s[j];
          cand[m].at = j;
          ++m;
        }
      }
      free(keep);
      qsort(pages, (size_t)n_keep_pages, sizeof(ranked), lower_index);
    }

    /* exact top-k of the candidates by a complete sort */
    qsort(cand, (size_t)m, sizeof(ranked), higher_key_then_lower_index);
    const int64_t k = m < topk ? m : topk;
    qsort(cand, (size_t)k, sizeof(ranked), lower_index);

    if (idx) {
      int32_t* out = idx + r * topk;
      for (int64_t t = 0; t < topk; ++t) out[t] = t < k ? (int32_t)cand[t].at : -1;
    }
    if (w) {
      float* out = w + r * topk;
      for (int64_t t = 0; t < topk; ++t) out[t] = t < k ? cand[t].key : 0.0f;
    }
    if (count) count[r] = (int32_t)k;
    if (page_mask) {
      uint64_t* out = page_mask + r * sh->max_pages;
      memset(out, 0, sizeof(uint64_t) * (size_t)sh->max_pages);
      for (int64_t t = 0; t < k; ++t) out[cand[t].at / bs] |= (uint64_t)1 << (cand[t].at % bs);
    }
    if (sel_pages && n_sel_pages > 0) {
      int32_t* out = sel_pages + r * n_sel_pages;
      for (int64_t t = 0; t < n_sel_pages; ++t)
        out[t] = t < n_keep_pages ? (int32_t)pages[t].at : -1;
    }
    free(pages);
    free(cand);
  }
  return 0;
}

/* -------------------------------------------------------------- attention */

int oracle_attend(const oracle_shape* sh, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* page_table, const int32_t* idx,
                  int32_t topk, double scale, double* out, double* lse, double* probs) {
  if (!shape_ok(sh) || sh->num_heads <= 0 || sh->head_dim <= 0 || !q || !k_cache ||
      !v_cache || !page_table || !idx || topk <= 0 || !out)
    return -1;
  const int64_t rows = (int64_t)sh->batch * sh->num_q;
  const int64_t limit = (int64_t)sh->max_pages * sh->block_size;
  const int H = sh->num_heads, D = sh->head_dim;
  const int hi = idx_heads(sh);
  if (H % hi != 0) return -1;
  const int group = H / hi; /* query heads per indexer head */
  for (int64_t t = 0; t < rows * hi * topk; ++t)
    if (idx[t] >= limit) return -1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
  for (int64_t r = 0; r < rows; ++r) {
    const int b = (int)(r / sh->num_q);
    double* logit = (double*)malloc(sizeof(double) * (size_t)topk);
    for (int h = 0; h < H; ++h) {
      /* query head h attends over the selection of indexer head h / group */
      const int32_t* sel = idx + (r * hi + h / group) * topk;
      const uint16_t* qh = q + (r * H + h) * D;
      double* o = out + (r * H + h) * D;
      double* ph = probs ? probs + (r * H + h) * topk : NULL;
      /* scaled logits of the selected positions */
      double mx = -INFINITY;
      int any = 0;
      for (int t = 0; t < topk; ++t) {
        if (sel[t] < 0) continue;
        const uint16_t* kr = k_cache + physical_row(sh, page_table, b, sel[t]) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += bf16_value(qh[d]) * bf16_value(kr[d]);
        logit[t] = scale * dot;
        if (!any || logit[t] > mx) mx = logit[t];
        any = 1;
      }
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (ph)
        for (int t = 0; t < topk; ++t) ph[t] = 0.0;
      if (!any) {
        if (lse) lse[r * H + h] = -INFINITY;
        continue;
      }
      /* softmax over the selected set, then the weighted sum of V rows */
      double z = 0.0;
      for (int t = 0; t < topk; ++t)
        if (sel[t] >= 0) z += exp(logit[t] - mx);
      for (int t = 0; t < topk; ++t) {
        if (sel[t] < 0) continue;
        const double pt = exp(logit[t] - mx) / z;
        if (ph) ph[t] = pt;
        const uint16_t* vr = v_cache + physical_row(sh, page_table, b, sel[t]) * D;
        for (int d = 0; d < D; ++d) o[d] += pt * bf16_value(vr[d]);
      }
      if (lse) lse[r * H + h] = mx + log(z);
    }
    free(logit);
  }
  return 0;
}

int oracle_dense_causal_attention(const oracle_shape* sh, const uint16_t* q,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* page_table, const int32_t* seq_lens,
                                  const int32_t* q_start, double scale,
                                  double* out, double* lse) {
  if (!shape_ok(sh) || sh->num_heads <= 0 || sh->head_dim <= 0 || !q || !k_cache ||
      !v_cache || !page_table || !out)
    return -1;
  if (!q_start && !seq_lens) return -1;
  const int64_t rows = (int64_t)sh->batch * sh->num_q;
  const int64_t limit = (int64_t)sh->max_pages * sh->block_size;
  const int H = sh->num_heads, D = sh->head_dim;
  for (int64_t r = 0; r < rows; ++r) {
    int64_t p = query_position(sh, seq_lens, q_start, (int)(r / sh->num_q), (int)(r % sh->num_q));
    if (p >= limit) return -1;
  }
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
  for (int64_t r = 0; r < rows; ++r) {
    const int b = (int)(r / sh->num_q), i = (int)(r % sh->num_q);
    const int64_t p = query_position(sh, seq_lens, q_start, b, i);
    const int64_t n = p >= 0 ? p + 1 : 0;
    double* weight = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int h = 0; h < H; ++h) {
      const uint16_t* qh = q + (r * H + h) * D;
      double* o = out + (r * H + h) * D;
      if (n == 0) {
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (lse) lse[r * H + h] = -INFINITY;
        continue;
      }
      /* pass 1: every causal logit, and their maximum */
      double top = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        const uint16_t* kr = k_cache + physical_row(sh, page_table, b, j) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += bf16_value(qh[d]) * bf16_value(kr[d]);
        weight[j] = scale * dot;
        if (weight[j] > top) top = weight[j];
      }
      /* pass 2: unnormalised weights and their total */
      double total = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        weight[j] = exp(weight[j] - top);
        total += weight[j];
      }
      /* pass 3: each output channel as a normalised weighted sum */
      for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j)
          acc += weight[j] * bf16_value(v_cache[physical_row(sh, page_table, b, j) * D + d]);
        o[d] = acc / total;
      }
      if (lse) lse[r * H + h] = top + log(total);
    }
    free(weight);
  }
  return 0;
}

int oracle_to_bf16(const double* in, uint16_t* out, int64_t n) {
  if ((!in || !out) && n > 0) return -1;
  for (int64_t t = 0; t < n; ++t) out[t] = fp32_to_bf16((float)in[t]);
  return 0;
}

/* ------------------------------------------------- MXFP4 -> FP8 conversion */

/* Value of an E2M1 code (OCP MX v1.0): bit 3 sign, bits 2-1 exponent with
 * bias 1, bit 0 mantissa; exponent field 0 encodes the subnormal 0.m * 2^0. */
static double e2m1_value(unsigned code) {
  const unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
  return s ? -mag : mag;
}

/* E4M3 (OCP FP8): bit 7 sign, bits 6-3 exponent with bias 7, bits 2-0
 * mantissa; exponent field 0 encodes the subnormals m/8 * 2^-6; field 15 with
 * mantissa 7 is NaN and there are no infinities, so the largest finite value
 * is 1.75 * 2^8 = 448. Round to nearest, ties to even; results beyond 448
 * saturate to 448 (everything from 448 up rounds to 448 or would round past
 * the largest finite code). */
static uint8_t e4m3_from_double(double v) {
  const uint8_t sign = signbit(v) ? 0x80u : 0x00u;
  if (isnan(v)) return (uint8_t)(sign | 0x7Fu);
  const double a = fabs(v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  if (a == 0.0) return sign;
  int e2;
  (void)frexp(a, &e2);
  int E = e2 - 1; /* a = m * 2^E with m in [1, 2) */
  if (E < -6) {
    /* subnormal range: a multiple of 2^-9, rounded half to even by rint
       (the default rounding mode); 8 * 2^-9 is the smallest normal 0x08 */
    const double k = rint(ldexp(a, 9));
    return (uint8_t)(sign | (uint8_t)k);
  }
  double q = rint((ldexp(a, -E) - 1.0) * 8.0);
  if (q == 8.0) {
    q = 0.0;
    E += 1;
  }
  return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | (int)q));
}

int oracle_mxfp4_to_fp8(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                        int64_t cols, int32_t exp_offset, uint8_t* out) {
  if (!packed || !scales || !out || rows < 0 || cols < 0 || cols % 32 != 0) return -1;
  if (exp_offset < -1024 || exp_offset > 1024) return -1;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      const uint8_t byte = packed[r * (cols / 2) + c / 2];
      const unsigned code = (c % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
      const unsigned x = scales[r * (cols / 32) + c / 32];
      const double e = e2m1_value(code);
      const double v = x == 255u ? copysign(NAN, e) : ldexp(e, (int)x - 127 + exp_offset);
      out[r * cols + c] = e4m3_from_double(v);
    }
  }
  return 0;
}

int oracle_mxfp4_to_fp8_experts(const uint8_t* packed, const uint8_t* scales,
                                int32_t num_experts, int64_t rows, int64_t cols,
                                const int32_t* expert_ids, int32_t n_sel,
                                int32_t exp_offset, uint8_t* out) {
  if (num_experts < 1 || n_sel < 0 || (n_sel > 0 && !expert_ids)) return -1;
  if (rows < 0 || cols < 0 || cols % 32 != 0) return -1;
  for (int32_t s = 0; s < n_sel; ++s) {
    const int32_t id = expert_ids[s];
    if (id < 0 || id >= num_experts) continue;
    const int rc = oracle_mxfp4_to_fp8(packed + (int64_t)id * rows * (cols / 2),
                                       scales + (int64_t)id * rows * (cols / 32), rows, cols,
                                       exp_offset, out + (int64_t)s * rows * cols);
    if (rc) return rc;
  }
  return 0;
}
