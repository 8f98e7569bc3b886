/*
 * oracle.h -- CPU oracle for index-selected sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library. It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * All pointers are host pointers. bf16 values are passed as their uint16 bit
 * pattern. Shapes use the same conventions as the GPU library's boundary so
 * that both sides can be handed the very same arrays:
 *   q_comp        bf16 [B][S_q][d_c]
 *   k_comp_cache  bf16 [P][bs][d_c]     (paged like K and V)
 *   k_cache       bf16 [P][bs][D]
 *   v_cache       bf16 [P][bs][D]
 *   q             bf16 [B][S_q][H][D]
 *   page_table    int32 [B][max_pages]  logical page -> physical page
 *   seq_lens      int32 [B]
 *   q_start       int32 [B] or NULL     query row i of sequence b sits at
 *                                       position q_start[b] + i; NULL means
 *                                       seq_lens[b] - S_q (the last rows)
 * Multi-head indexer ("Day-0 Inference Adaptation of Ultra-Large-Scale MoE
 * Models on Domestic AI Accelerators", section 4.1: scores shaped
 * [B, H, S, S_c] and a top-k along the last axis): with Hi indexer heads,
 * q_comp is [B][S_q][Hi][d_c] and every (query row, indexer head) is a
 * selection row of its own, at the query row's position, over the one shared
 * compressed key per position; scores, idx, w, count and page_mask gain the
 * Hi axis after S_q. Query head h attends over the selection of indexer
 * head h / (H / Hi). Hi = 1 is the single shared indexer head.
 * Every function returns 0, or -1 for an argument it cannot use.
 */
#ifndef TIS_ORACLE_H
#define TIS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_shape {
  int32_t batch;      /* B */
  int32_t num_q;      /* S_q */
  int32_t d_c;        /* indexer width */
  int32_t num_heads;  /* H query heads sharing one KV head */
  int32_t head_dim;   /* D */
  int32_t block_size; /* bs: tokens per page */
  int32_t max_pages;  /* page-table row stride */
  int32_t num_idx_heads; /* Hi indexer heads (0 is read as 1); Hi divides H */
} oracle_shape;

int oracle_set_threads(int n);
int oracle_get_threads(void);

/* s[j] = sum_c q_comp[c] * k_comp[j][c] for every j <= p, summed in fp64 and
 * rounded once to fp32. scores is [B][S_q][ld]; entries j > p are untouched. */
int oracle_index_scores(const oracle_shape* sh, const uint16_t* q_comp,
                        const uint16_t* k_comp_cache, const int32_t* page_table,
                        const int32_t* seq_lens, const int32_t* q_start,
                        float* scores, int64_t ld);

/* Masked top-k with the key (score descending, position ascending).
 * n_sel_pages == 0: candidates are all positions j <= p.
 * n_sel_pages  > 0: page maxima over valid positions, the first n_sel_pages
 *                   pages by (max descending, page ascending), candidates are
 *                   the valid positions inside them.
 * Outputs per row (each may be NULL):
 *   idx       int32 [B][S_q][topk]  ascending positions, -1 padded
 *   w         fp32  [B][S_q][topk]  score of each selected position, 0 padded
 *   count     int32 [B][S_q]        number selected
 *   page_mask u64   [B][S_q][max_pages]  bit t of word g <=> g*bs+t selected
 *   sel_pages int32 [B][S_q][n_sel_pages] ascending logical pages, -1 padded
 */
int oracle_topk_select(const oracle_shape* sh, const float* scores, int64_t ld,
                       const int32_t* seq_lens, const int32_t* q_start,
                       int32_t topk, int32_t n_sel_pages,
                       int32_t* idx, float* w, int32_t* count,
                       uint64_t* page_mask, int32_t* sel_pages);

/* Exact softmax attention of each query head over the positions listed in
 * idx (entries < 0 are skipped), computed in fp64.
 *   out   fp64 [B][S_q][H][D]
 *   lse   fp64 [B][S_q][H]      natural-log sum of exp of the scaled logits
 *   probs fp64 [B][S_q][H][topk] softmax weight of each idx entry (0 for
 *         skipped entries); may be NULL
 * A row with no valid entry gets out = 0 and lse = -inf. */
int oracle_attend(const oracle_shape* sh, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* page_table, const int32_t* idx,
                  int32_t topk, double scale, double* out, double* lse, double* probs);

/* Dense causal attention over every position j <= p, coded separately from
 * oracle_attend (no index list). Same output layout. */
int oracle_dense_causal_attention(const oracle_shape* sh, const uint16_t* q,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* page_table, const int32_t* seq_lens,
                                  const int32_t* q_start, double scale,
                                  double* out, double* lse);

/* fp64 -> fp32 -> bf16, rounding to nearest even at the second step. */
int oracle_to_bf16(const double* in, uint16_t* out, int64_t n);

/* Online conversion of MXFP4 expert weights to FP8 E4M3 ("Day-0 Inference
 * Adaptation for Ultra-Large MoE Models on Domestic GPUs", section "Handling
 * Low-Precision Expert Weights: Online Conversion and Workspace Reuse"; "Day-0
 * Adaptation for Trillion-Parameter MoE Models", section V).
 * A weight matrix is [rows][cols], cols a multiple of 32:
 *   packed  u8 [rows][cols/2]   two E2M1 elements per byte: element 2i in
 *                               bits 0-3 of byte i, element 2i+1 in bits 4-7
 *   scales  u8 [rows][cols/32]  one E8M0 scale per 32 consecutive elements
 *                               of a row (value 2^(X-127); X = 255 is NaN)
 *   out     u8 [rows][cols]     FP8 E4M3 bit patterns of
 *                               2^exp_offset * 2^(X-127) * element,
 *                               rounded to nearest (ties to even), finite
 *                               results above 448 saturated to 448, zeros and
 *                               NaNs keeping the element's sign.
 * Formats: OCP Microscaling Formats (MX) v1.0 (E2M1, E8M0) and OCP 8-bit
 * Floating Point (E4M3). |exp_offset| <= 1024. */
int oracle_mxfp4_to_fp8(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                        int64_t cols, int32_t exp_offset, uint8_t* out);

/* The conversion for the experts a router selected: slot s of out
 * ([n_sel][rows][cols]) receives expert expert_ids[s] of the weight pool
 * (packed [num_experts][rows][cols/2], scales [num_experts][rows][cols/32]).
 * A slot whose id lies outside [0, num_experts) is left unchanged. */
int oracle_mxfp4_to_fp8_experts(const uint8_t* packed, const uint8_t* scales,
                                int32_t num_experts, int64_t rows, int64_t cols,
                                const int32_t* expert_ids, int32_t n_sel,
                                int32_t exp_offset, uint8_t* out);

#ifdef __cplusplus
}
#endif
#endif
