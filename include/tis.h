/*
 * tis.h -- index-selected sparse attention on MI355X (gfx950): the C ABI.
 *
 * The method (three pages on one subject):
 *  - "Day-0 Inference Adaptation of Ultra-Large-Scale MoE Models on Domestic AI
 *    Accelerators", section 4.1 "Sparse Attention Index Pipeline": score
 *    compressed query/key representations, select the top-k positions per query
 *    on the device, gather the full K/V rows of those positions, and run exact
 *    attention over them only.
 *  - "Day-0 Inference Adaptation for Ultra-Large MoE Models on Domestic GPUs: A
 *    Software Stack Perspective", sections "Operatorizing Index Selection"
 *    (scoring, top-k and masking fused; block-level pruning then exact selection
 *    inside the kept blocks), "Reorganizing KV Cache Layout" (a block-organised
 *    KV cache addressed by block ids) and "Separate Paths for Prefill and
 *    Decode" (separate schedules sharing one sparse-mask representation).
 *  - "Day-0 Adaptation for Trillion-Parameter MoE Models: A Comprehensive Guide
 *    to Heterogeneous Compute Deployment", section IV (page-table KV layout;
 *    prefill and decode as two kernels; retrieval pipelined with attention).
 *
 * Conventions shared by every entry point
 *  - Every array argument is a DEVICE pointer unless a comment says "host".
 *    bf16 arrays are passed as their uint16 bit patterns.
 *  - The caller allocates and owns every buffer, including the workspace; the
 *    library allocates nothing, frees nothing and keeps no pointer after a call
 *    returns.
 *  - Work is enqueued on `stream` (a hipStream_t cast to void*; NULL = the
 *    default stream) and calls return once it is enqueued. Buffers and the
 *    workspace must stay alive until the stream has passed the work. Calls that
 *    share a workspace must be ordered on one stream.
 *  - Return value: TIS_OK, or a negative TIS_ERR_* code. Arguments are checked
 *    before anything is enqueued; on an error nothing is launched and
 *    tis_last_error() describes it. Device faults surface at the caller's
 *    synchronisation, as for any HIP kernel.
 *  - Supported sizes: d_c 64 or 128; head_dim 128; block_size 64;
 *    1 <= num_heads <= 64; 1 <= num_idx_heads <= 16 dividing num_heads;
 *    1 <= topk <= 4096; 0 <= n_sel_pages <= 192.
 *    Other values return TIS_ERR_UNSUPPORTED.
 *  - Results are bitwise deterministic for identical inputs on one device.
 *
 * Common tensors
 *   q_comp        bf16  [B][S_q][d_c]      compressed query rows
 *   k_comp_cache  bf16  [P][bs][d_c]       compressed keys, paged like K and V
 *   k_cache       bf16  [P][bs][D]         keys
 *   v_cache       bf16  [P][bs][D]         values
 *   q             bf16  [B][S_q][H][D]     query heads; all H share one KV head
 *   page_table    int32 [B][max_pages]     logical page g of sequence b lives in
 *                                          physical page page_table[b][g]; position
 *                                          j is slot j % bs of logical page j / bs
 *   seq_lens      int32 [B]                tokens held for each sequence
 *   q_start       int32 [B] or NULL        query row i of sequence b sits at
 *                                          position p = q_start[b] + i; NULL means
 *                                          q_start[b] = seq_lens[b] - S_q
 *   Query row i of sequence b attends causally to positions 0..p (inclusive).
 *
 * Indexer heads ("Sparse Attention Index Pipeline", section 4.1: the scores
 * are shaped [B, H, S, S_c] and the top-k runs along the last axis). With
 * Hi = num_idx_heads > 1 every (query row, indexer head) is a selection row
 * of its own, at the query row's position, scored against the one compressed
 * key per position that all heads share:
 *   q_comp                          bf16 [B][S_q][Hi][d_c]
 *   scores                          fp32 [B][S_q][Hi][ld_scores]
 *   idx, w                          [B][S_q][Hi][topk]
 *   count                           int32 [B][S_q][Hi]
 *   page_mask                       u64 [B][S_q][Hi][max_pages_per_seq]
 * and query head h attends over the selection of indexer head h / (H / Hi)
 * (q, out and lse keep their [B][S_q][H] layout). Hi = 1 is one indexer head
 * shared by all query heads, and the layouts above lose the Hi axis.
 *   The caller guarantees p < seq_lens[b] <= max_pages * bs and page ids in
 *   [0, num_phys_pages). A row with p < 0 (in decode: a sequence that holds no
 *   tokens yet, seq_lens[b] == 0) has no candidates: it selects nothing
 *   (count 0, idx all -1, w 0, an empty page mask) and its attention output is
 *   0 with lse -inf. Kernels clamp out-of-range positions and page ids so that
 *   no access leaves the arrays; results are then unspecified.
 */
#ifndef TIS_H
#define TIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TIS_ABI_VERSION 2

enum {
  TIS_OK = 0,
  TIS_ERR_INVALID_ARG = -1,         /* null pointer, negative size, bad enum     */
  TIS_ERR_UNSUPPORTED = -2,         /* a size outside the supported set          */
  TIS_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes < tis_workspace_size(...) */
  TIS_ERR_HIP = -4                  /* a HIP launch or runtime call failed       */
};

enum { TIS_PHASE_DECODE = 0, TIS_PHASE_PREFILL = 1 };

/* ops for tis_workspace_size */
enum {
  TIS_OP_INDEX_SCORE = 0,
  TIS_OP_TOPK_SELECT = 1, /* with scores == NULL (scoring fused in)            */
  TIS_OP_TOPK_SELECT_GIVEN_SCORES = 2,
  TIS_OP_GATHER_ATTEND_DECODE = 3,
  TIS_OP_GATHER_ATTEND_PREFILL = 4,
  TIS_OP_DECODE_STEP = 5
};

/* Problem sizes; a host struct read during the call only. */
typedef struct tis_shape {
  int32_t batch;             /* B                                               */
  int32_t num_q;             /* S_q query rows per sequence (1 for decode)      */
  int32_t d_c;               /* indexer width: 64 or 128 (one shared head)      */
  int32_t num_heads;         /* H query heads sharing one KV head               */
  int32_t head_dim;          /* D: 128                                          */
  int32_t block_size;        /* bs tokens per page: 64                          */
  int32_t max_pages_per_seq; /* page_table row stride; times bs below 2^31-2^20 */
  int32_t num_phys_pages;    /* P, pages in each cache pool                     */
  int32_t num_idx_heads;     /* Hi indexer heads, 1..16 dividing num_heads (0 is
                                read as 1); see "Indexer heads" above         */
} tis_shape;

/* Indexer scores ("Sparse Attention Index Pipeline", section 4.1, step 1:
 * scores = q_comp . k_comp^T over the causal context).
 *   scores  fp32 [B][S_q][ld_scores]; entry j of row (b, i) receives
 *           sum_c q_comp[b][i][c] * k_comp[j][c] for j <= p, accumulated in
 *           fp32 from bf16 inputs; entries j > p are not written.
 *   ld_scores >= max_pages_per_seq * block_size.
 * No workspace. S_q == 1 runs the decode (bandwidth-bound) scorer, S_q > 1 the
 * prefill scorer on MFMA tiles. */
int sparse_index_score(const tis_shape* shape, const uint16_t* q_comp,
                       const uint16_t* k_comp_cache, const int32_t* page_table,
                       const int32_t* seq_lens, const int32_t* q_start, float* scores,
                       int64_t ld_scores, void* stream);

/* Masked top-k index selection ("Operatorizing Index Selection": scoring, top-k
 * and masking in one operator; section 4.1 step 2: top-k positions and their
 * scores).
 *   scores       fp32 [B][S_q][ld_scores] from sparse_index_score, or NULL to
 *                compute them inside the call (into the workspace).
 *   topk         positions kept per row; a row with fewer than topk candidates
 *                keeps them all.
 *   n_sel_pages  0: candidates are every position j <= p.
 *                >0: block pruning first: the n_sel_pages pages with the largest
 *                maximum score over their valid positions are kept (ties: lower
 *                logical page), and the top-k is taken among their positions.
 * Selection key: higher score first, then lower position (-0.0 equals +0.0).
 * Outputs (each may be NULL except idx):
 *   idx        int32 [B][S_q][topk]   selected positions in ascending order,
 *                                     then -1 padding
 *   w          fp32  [B][S_q][topk]   the selected scores (0 padding)
 *   count      int32 [B][S_q]         number selected
 *   page_mask  u64   [B][S_q][max_pages_per_seq]  bit t of word g is set iff
 *              position g*bs + t is selected: the sparse-mask representation
 *              shared by the prefill and decode attention paths.
 * Needs tis_workspace_size(shape, TIS_OP_TOPK_SELECT or
 * TIS_OP_TOPK_SELECT_GIVEN_SCORES, topk, n_sel_pages) bytes of workspace. */
int sparse_topk_select(const tis_shape* shape, const uint16_t* q_comp,
                       const uint16_t* k_comp_cache, const float* scores,
                       int64_t ld_scores, const int32_t* page_table,
                       const int32_t* seq_lens, const int32_t* q_start, int32_t topk,
                       int32_t n_sel_pages, int32_t* idx, float* w, int32_t* count,
                       uint64_t* page_mask, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Gather the selected K/V rows through the page table and run exact softmax
 * attention over them ("Sparse Attention Index Pipeline", section 4.1 step 3;
 * section IV's two-phase sparse attention).
 *   phase   TIS_PHASE_DECODE: each row's selection is split across workgroups and
 *           the partial softmax states are merged. TIS_PHASE_PREFILL: a
 *           workgroup takes a run of consecutive query rows, turns their index
 *           lists into the per-(row, page) bitmask and streams every page any of
 *           them selected through on-chip memory once, in windows of 128 pages
 *           for longer contexts. Where the rows' contexts average more than
 *           4 * topk positions (a sparse selection; the rows are taken to end at
 *           the longest context) the per-row gather of the decode phase is used.
 *   idx     int32 [B][S_q][topk] as produced by sparse_topk_select; entries < 0
 *           are skipped. The non-negative entries of a row must be distinct
 *           positions (as sparse_topk_select produces them): the prefill phase
 *           works from the bitmask, where a repeated position counts once.
 *   softmax_scale  logits are softmax_scale * q.k; <= 0 selects 1/sqrt(head_dim).
 *   out     bf16 [B][S_q][H][D]: sum_j softmax(logits)_j * v_j (fp32
 *           accumulation, round to nearest even). A row with no selected
 *           position gets zeros.
 *   lse     fp32 [B][S_q][H] natural-log sum of exp of the logits (-inf for an
 *           empty row), or NULL.
 * Needs tis_workspace_size(shape, TIS_OP_GATHER_ATTEND_DECODE or _PREFILL, topk,
 * 0) bytes of workspace (zero for prefill). */
int paged_gather_attend(const tis_shape* shape, int32_t phase, const uint16_t* q,
                        const uint16_t* k_cache, const uint16_t* v_cache,
                        const int32_t* page_table, const int32_t* idx, int32_t topk,
                        float softmax_scale, uint16_t* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* One fused decode step (S_q must be 1): scoring, masked top-k (or block-pruned
 * top-k), gather and attention for the query at p = seq_lens[b] - 1 of every
 * sequence ("Separate Paths for Prefill and Decode": the decode path).
 *   out   bf16 [B][1][H][D]
 *   idx   int32 [B][1][topk] or NULL;  w fp32 [B][1][topk] or NULL;
 *   lse   fp32 [B][1][H] or NULL.
 * Needs tis_workspace_size(shape, TIS_OP_DECODE_STEP, topk, n_sel_pages) bytes. */
int sparse_decode_step(const tis_shape* shape, const uint16_t* q_comp,
                       const uint16_t* k_comp_cache, const uint16_t* q,
                       const uint16_t* k_cache, const uint16_t* v_cache,
                       const int32_t* page_table, const int32_t* seq_lens, int32_t topk,
                       int32_t n_sel_pages, float softmax_scale, uint16_t* out,
                       int32_t* idx, float* w, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);

/* sparse_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results without a workspace. Its
 * scratch memory is a fixed 64 MiB array in device memory, one per device,
 * held from the library's load on that device until the process ends; the
 * call uses the array of the current device, and `stream` must belong to
 * that device. The call allocates nothing. Shapes whose workspace
 * (tis_workspace_size with TIS_OP_DECODE_STEP) exceeds 64 MiB return
 * TIS_ERR_UNSUPPORTED before anything is launched. Every call on a device
 * shares its array: calls that may overlap on one device (different streams,
 * threads or processes without ordering) race and must be serialised by the
 * caller. The array keeps the last call's contents; each call clears what it
 * needs cleared with kernels of its own (no memset). */
int sparse_decode_step_noalloc(const tis_shape* shape, const uint16_t* q_comp,
                               const uint16_t* k_comp_cache, const uint16_t* q,
                               const uint16_t* k_cache, const uint16_t* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, int32_t topk,
                               int32_t n_sel_pages, float softmax_scale, uint16_t* out,
                               int32_t* idx, float* w, float* lse, void* stream);

/* Append one token per sequence to the paged caches: the rows are written at
 * position seq_lens[b] (page seq_lens[b] / bs of the page table, slot
 * seq_lens[b] % bs) and seq_lens[b] is incremented on the device. A sequence
 * whose cache is full (seq_lens[b] == max_pages * bs) is left unchanged.
 * ("Reorganizing KV Cache Layout": one block-level cache shared by prefill and
 * decode.)
 *   k_comp_new bf16 [B][d_c], k_new bf16 [B][D], v_new bf16 [B][D]. */
int paged_kv_append(const tis_shape* shape, const uint16_t* k_comp_new,
                    const uint16_t* k_new, const uint16_t* v_new,
                    const int32_t* page_table, int32_t* seq_lens, uint16_t* k_comp_cache,
                    uint16_t* k_cache, uint16_t* v_cache, void* stream);

/* Online conversion of low-precision expert weights ("Day-0 Inference
 * Adaptation for Ultra-Large MoE Models on Domestic GPUs", section "Handling
 * Low-Precision Expert Weights: Online Conversion and Workspace Reuse"; "Day-0
 * Adaptation for Trillion-Parameter MoE Models", section V): the MXFP4
 * weights of the experts a router selected are dequantised into FP8 E4M3 in
 * a caller-owned working buffer, which the caller reuses from layer to layer.
 *   w_packed    u8 [num_experts][rows][cols/2]: the MXFP4 (E2M1) elements of
 *               each expert's [rows][cols] weight matrix, two per byte,
 *               element 2i in bits 0-3 of byte i (8-byte aligned)
 *   w_scales    u8 [num_experts][rows][cols/32]: one E8M0 scale 2^(X-127) per
 *               32 consecutive elements of a row (X = 255: NaN)
 *   expert_ids  int32 [n_sel], device memory: slot s of fp8_out receives
 *               expert expert_ids[s]; an id outside [0, num_experts) leaves
 *               its slot unwritten
 *   exp_offset  every value is also multiplied by 2^exp_offset (0: the plain
 *               dequantised values); |exp_offset| <= 1024
 *   fp8_out     u8 [n_sel][rows][cols] E4M3 bit patterns (16-byte aligned),
 *               out_bytes >= n_sel * rows * cols; slots from n_sel on are not
 *               touched
 * Each value e * 2^(X-127+exp_offset) is rounded to the nearest E4M3 value,
 * ties to even; finite results above 448 saturate to 448; zeros and NaNs keep
 * the element's sign. Formats: OCP Microscaling (MX) v1.0 and OCP FP8 E4M3.
 * cols must be a multiple of 32 (else TIS_ERR_UNSUPPORTED); n_sel <= 65535;
 * n_sel == 0 launches nothing. No workspace. */
int mxfp4_to_fp8_experts(const uint8_t* w_packed, const uint8_t* w_scales, int32_t num_experts,
                         int32_t rows, int32_t cols, const int32_t* expert_ids, int32_t n_sel,
                         int32_t exp_offset, uint8_t* fp8_out, size_t out_bytes, void* stream);

/* Workspace bytes an entry point needs for `shape` (0 when it needs none, or
 * for an invalid request; tis_last_error() then says why). */
size_t tis_workspace_size(const tis_shape* shape, int32_t op, int32_t topk,
                          int32_t n_sel_pages);

/* Message for the last nonzero return on the calling thread ("" if none). */
const char* tis_last_error(void);

/* TIS_ABI_VERSION of the loaded library. */
int tis_abi_version(void);

/* Stage timing, for benchmarks and profiling. While enabled (on != 0), every
 * entry point records a pair of HIP events on its stream around each kernel
 * launch. tis_stage_timing_read waits for the recorded work, writes the
 * accumulated milliseconds and launch counts per stage into host arrays of at
 * least TIS_NUM_STAGES entries (index = stage id, see tis_stage_name), and
 * clears the records. tis_stage_timing_enable returns the previous setting.
 * Stages: 0 histogram clear, 1 scorer, 2 first-digit histogram, 3 candidate
 * collection, 4 select, 5 gather-attend, 6 split combine, 7 cache append,
 * 8 MXFP4 -> FP8 conversion. */
#define TIS_NUM_STAGES 9
int tis_stage_timing_enable(int on);
int tis_stage_timing_read(double* ms, int64_t* launches, int32_t n_stages);
const char* tis_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif
#endif /* TIS_H */
