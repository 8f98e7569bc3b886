// tis_internal.h -- host-side launchers shared between the translation units of
// libtis. Internal; not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tis {

// Rows of n positions or fewer are selected straight from an LDS copy of the
// row; longer rows go through the histogram + candidate path.
constexpr int kDecodeKeyCap = 12288;
constexpr int kDecodePosCap = 12288;
// Threads of a selection block: prefill rows run three 512-thread blocks per
// CU (six waves per SIMD); a decode row's block holds the large key and
// position buffers alone on its CU and takes 1024 threads.
constexpr int kPrefillSelectThreads = 512;
constexpr int kDecodeSelectThreads = 1024;
constexpr int kPrefillKeyCap = 8192;
// Pages per block of the decode scorer without histograms: 16, or 4 (one page
// per wave) when even 16-page blocks would leave compute units idle, so that a
// short launch's waves each walk fewer pages in sequence.
constexpr int kPagesPerScoreBlock = 16;
constexpr int kPagesPerScoreBlockSmall = 4;
// Pages per block of the histogramming decode scorer: 24 when a launch runs
// several rounds of blocks (its tail is then shorter), 32 when one round of
// such blocks covers every row (few long rows: fewer blocks then add into the
// same row histogram).
constexpr int kPagesPerHistScoreBlockNarrow = 24;
constexpr int kPagesPerHistScoreBlockWide = 32;
// The page-maxima decode scorer that holds a block's scores in LDS until the
// block ends: at most this many pages per block (32 KiB of scores), and used
// when the table gives blocks of at least kMinDeferPages in one round.
constexpr int kMaxDeferPages = 128;
constexpr int kMinDeferPages = 16;
constexpr int kAttendTile = 32;             // keys per attention tile
constexpr int kMaxSplits = 256;             // decode splits per row (combine: one per thread)

constexpr int kHistChunk = 16384;   // positions per histogram block
constexpr int kHistThreads = 1024;  // threads per histogram block

struct ScoreDecodeArgs {
  const uint16_t* q_comp;
  const uint16_t* k_comp;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_start;
  int batch, d_c, max_pages, num_phys;
  float* scores;     // [B][hq][ld]
  int64_t ld;
  int hq;            // indexer heads (selection rows per sequence)
  float* page_max;   // [B][hq][max_pages] or null
  uint32_t* row_hist;  // [B][kRowHistWords] zeroed first-digit histograms to add into, or null
  int64_t long_row_min;  // rows with at least this many positions are histogrammed
  int ppb;             // pages per block (set by the launcher)
};
hipError_t launch_score_decode(const ScoreDecodeArgs& a, hipStream_t s);

struct ScorePrefillArgs {
  const uint16_t* q_comp;
  const uint16_t* k_comp;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_start;
  int batch, num_q, d_c, max_pages, num_phys;
  float* scores;   // [B][num_q][hq][ld]
  int64_t ld;
  int hq;          // indexer heads: row r of a sequence is query row r / hq
  int skip_n;      // > 0: blocks whose rows all see at most skip_n positions write
                   // nothing (the selection keeps all of such a row unread)
};
hipError_t launch_score_prefill(const ScorePrefillArgs& a, hipStream_t s);

constexpr int kCollectBlock = 4096;  // positions per candidate slice
// Compute units of the current device (queried once per device).
int device_cus();

struct HistArgs {  // first-digit histograms of long decode rows
  const float* scores;
  int64_t ld;
  const int32_t* seq_lens;
  const int32_t* q_start;
  int rows, hq, max_pages;  // selection rows (batch * hq); row r is of sequence r / hq
  uint32_t* row_hist;  // [rows][kRowHistWords], cleared before launch_hist
  int64_t long_row_min;
};
hipError_t launch_hist_clear(const HistArgs& a, hipStream_t s);
hipError_t launch_hist(const HistArgs& a, hipStream_t s);

struct CollectArgs {  // threshold digit and candidate slices of long decode rows
  const float* scores;
  int64_t ld;
  const int32_t* seq_lens;
  const int32_t* q_start;
  int rows, hq, max_pages, topk;  // selection rows; row r is of sequence r / hq
  const uint32_t* row_hist;  // [rows][kRowHistWords] complete first-digit histograms (fine, coarse)
  int32_t* thresh;           // [rows] first digit of the K'-th largest key
  int32_t* above;            // [rows] number of keys whose first digit exceeds it
  int64_t long_row_min;
  uint32_t* cand_key;        // [rows][cand_ld]: slice s starts at s * kCollectBlock
  int32_t* cand_pos;
  int64_t cand_ld;
  int32_t* slice_cnt;        // [rows][slice_ld]
  int slice_ld;
};
hipError_t launch_collect(const CollectArgs& a, hipStream_t s);

struct SelectArgs {
  const float* scores;
  int64_t ld;
  const int32_t* seq_lens;
  const int32_t* q_start;
  // selection rows: batch * num_q * hq; row r is query row (r / hq) % num_q
  // of sequence r / (num_q * hq)
  int batch, num_q, hq, max_pages, topk, n_sel_pages;
  const float* page_max;   // [rows][max_pages] or null
  const uint32_t* cand_key;  // long rows: candidate slices from collect (or null)
  const int32_t* cand_pos;
  const int32_t* slice_cnt;
  const int32_t* thresh;
  const int32_t* above;
  int64_t cand_ld;
  int slice_ld;
  int64_t long_row_min;    // rows with n >= this use the candidates (if given)
  int32_t* idx;
  float* w;
  int32_t* count;
  uint64_t* page_mask;
};
hipError_t launch_select(const SelectArgs& a, bool prefill_rows, hipStream_t s);

struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* idx;          // [rows][topk]
  // rows: selection rows B * S_q * idx_heads; row r is query row
  // (r / idx_heads) % num_q of sequence r / (num_q * idx_heads), and its
  // num_heads query heads (those of indexer head r % idx_heads) are q and out
  // rows r * num_heads ...
  int rows, num_q, idx_heads, num_heads, max_pages, num_phys, topk;
  float scale;
  int keys_per_split, n_splits;
  int head_groups;  // waves per (row, split), each taking its own head tiles
  uint16_t* out;
  float* lse;
  float* part_o;   // [rows*n_splits][num_heads][D]
  float* part_ml;  // [rows*n_splits][num_heads][3]: max, bf16-weight sum, fp32 sum
};
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

// Prefill attention over the per-(row, page) bitmask of consecutive query rows
// (pages streamed through LDS once per group of rows); the bitmask covers a
// window of kPrefillMaskPages pages at a time.
constexpr int kPrefillMaskPages = 128;
bool prefill_attend_supported(int max_pages, int num_q, int num_heads, int topk);
hipError_t launch_prefill_attend(const AttendArgs& a, int batch, hipStream_t s);
hipError_t launch_combine(const AttendArgs& a, hipStream_t s);  // no-op for one split

// Online MXFP4 -> FP8 E4M3 conversion of router-selected expert weights
struct Mxfp4Args {
  const uint8_t* packed;      // [num_experts][rows][cols/2]
  const uint8_t* scales;      // [num_experts][rows][cols/32]
  int num_experts;
  int64_t rows, cols;         // cols a multiple of 32
  const int32_t* expert_ids;  // [n_sel] (device)
  int n_sel, exp_offset;
  uint8_t* out;               // [n_sel][rows][cols]
};
hipError_t launch_mxfp4_to_fp8(const Mxfp4Args& a, hipStream_t s);

struct AppendArgs {
  const uint16_t* k_comp_new;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* page_table;
  int32_t* seq_lens;
  uint16_t* k_comp_cache;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int batch, d_c, max_pages, num_phys;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

}  // namespace tis
