// api.hip -- the C ABI of libtis: argument checks, workspace plans and the
// launch sequences of the prefill and decode paths.
//
// Decode path ("Separate Paths for Prefill and Decode": memory-bound, one token
// per sequence): decode scorer (+ page maxima) -> [first-digit histogram ->
// threshold digit and candidate collection, for rows longer than the LDS select
// holds] -> select -> gather-attend split over waves -> combine. Prefill path
// (compute-bound): MFMA scorer -> select, one block per query row -> block-sparse
// attention over the per-(row, page) bitmask, a run of query rows per workgroup.
// Both paths produce the same index list and page bitmask.
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "tis.h"
#include "tis_common.h"
#include "tis_internal.h"

using namespace tis;

namespace {

thread_local std::string g_error;

int fail(int code, const std::string& msg) {
  g_error = msg;
  return code;
}

int ok() {
  g_error.clear();
  return TIS_OK;
}

constexpr int kMaxTopk = 4096;
constexpr int kMaxSelPages = 192;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// indexer heads: every (query row, indexer head) is one selection row
int idx_heads(const tis_shape* s) { return s->num_idx_heads > 1 ? s->num_idx_heads : 1; }

// selection rows of a call: B * S_q * Hi
int64_t sel_rows(const tis_shape* s) { return (int64_t)s->batch * s->num_q * idx_heads(s); }

int check_shape(const tis_shape* s) {
  if (!s) return fail(TIS_ERR_INVALID_ARG, "shape is NULL");
  if (s->num_idx_heads < 0) return fail(TIS_ERR_INVALID_ARG, "num_idx_heads must be >= 0");
  if (s->num_idx_heads > 16) return fail(TIS_ERR_UNSUPPORTED, "num_idx_heads must be <= 16");
  if (s->batch < 1 || s->num_q < 1 || s->max_pages_per_seq < 1 || s->num_phys_pages < 1 ||
      s->num_heads < 1)
    return fail(TIS_ERR_INVALID_ARG,
                "batch, num_q, num_heads, max_pages_per_seq and num_phys_pages must be >= 1");
  if (s->d_c != 64 && s->d_c != 128) return fail(TIS_ERR_UNSUPPORTED, "d_c must be 64 or 128");
  if (s->head_dim != kHeadDim) return fail(TIS_ERR_UNSUPPORTED, "head_dim must be 128");
  if (s->block_size != kBlockSize) return fail(TIS_ERR_UNSUPPORTED, "block_size must be 64");
  if (s->num_heads > 64) return fail(TIS_ERR_UNSUPPORTED, "num_heads must be <= 64");
  if (s->batch > 65535) return fail(TIS_ERR_UNSUPPORTED, "batch must be <= 65535");
  // positions are 32-bit in the kernels, with room for a block's stride past the end
  if ((int64_t)s->max_pages_per_seq * kBlockSize > (int64_t)INT32_MAX - (1 << 20))
    return fail(TIS_ERR_UNSUPPORTED, "max_pages_per_seq * block_size must be below 2^31 - 2^20");
  if ((int64_t)s->num_q > (int64_t)65535 * 64)
    return fail(TIS_ERR_UNSUPPORTED, "num_q must be <= 4194240");
  if (s->num_heads % idx_heads(s) != 0)
    return fail(TIS_ERR_UNSUPPORTED, "num_idx_heads must divide num_heads");
  const int64_t rows = sel_rows(s);
  if (rows > (int64_t)INT32_MAX / 64)
    return fail(TIS_ERR_UNSUPPORTED, "batch * num_q * num_idx_heads too large");
  if (idx_heads(s) > 1 && s->num_q == 1 && rows > 65535)
    return fail(TIS_ERR_UNSUPPORTED, "decode with several indexer heads: batch * num_idx_heads "
                                     "must be <= 65535");
  return TIS_OK;
}

int check_topk(int32_t topk, int32_t n_sel_pages) {
  if (topk < 1) return fail(TIS_ERR_INVALID_ARG, "topk must be >= 1");
  if (topk > kMaxTopk) return fail(TIS_ERR_UNSUPPORTED, "topk must be <= 4096");
  if (n_sel_pages < 0) return fail(TIS_ERR_INVALID_ARG, "n_sel_pages must be >= 0");
  if (n_sel_pages > kMaxSelPages) return fail(TIS_ERR_UNSUPPORTED, "n_sel_pages must be <= 192");
  return TIS_OK;
}

// ------------------------------------------------------------ workspace plan

struct Plan {
  int64_t rows = 0, cap = 0;
  bool prefill_rows = false, own_scores = false, long_rows = false, pmax = false;
  bool own_idx = false, attend_decode = false;
  int keys_per_split = 0, n_splits = 1;
  int slice_ld = 0;
  size_t off_scores = 0, off_pmax = 0, off_hist = 0, off_thresh = 0, off_above = 0;
  size_t off_ckey = 0, off_cpos = 0, off_slice = 0, off_idx = 0, off_po = 0, off_pml = 0;
  size_t total = 0;
};

void split_plan(const tis_shape* s, int32_t topk, bool decode, Plan* p) {
  const int64_t rows = sel_rows(s);
  const int tiles = (topk + kAttendTile - 1) / kAttendTile;
  if (!decode) {
    p->keys_per_split = tiles * kAttendTile;
    p->n_splits = 1;
    return;
  }
  // Splits of 32-key tiles, doubled while the launch keeps enough units to
  // cover the machine (>= 1024 (row, split) units), and up to 4 tiles while it
  // keeps at least one wave per CU (a wave per (row, split, 16-head group)):
  // few long rows then merge fewer partial states (block pruning over 8 rows:
  // 11.8 -> 9.8 us) without leaving CUs idle (the one-row stream keeps 1 tile).
  const int64_t head_groups = (s->num_heads / idx_heads(s) + 15) / 16;
  auto splits = [&](int k) { return (int64_t)((topk + k - 1) / k); };
  int kps = kAttendTile;
  while (kps * 2 <= tiles * kAttendTile &&
         (rows * splits(kps * 2) >= 1024 ||
          (kps * 2 <= 4 * kAttendTile && rows * splits(kps * 2) * head_groups >= device_cus())))
    kps *= 2;
  p->keys_per_split = kps;
  p->n_splits = (topk + kps - 1) / kps;
}

// select: scores_given / decode attend / own idx
Plan make_plan(const tis_shape* s, int32_t op, int32_t topk, int32_t n_sel_pages) {
  Plan p;
  p.rows = sel_rows(s);
  p.cap = (int64_t)s->max_pages_per_seq * kBlockSize;
  p.prefill_rows = s->num_q > 1;
  const bool select = op == TIS_OP_TOPK_SELECT || op == TIS_OP_TOPK_SELECT_GIVEN_SCORES ||
                      op == TIS_OP_DECODE_STEP;
  const bool attend_decode = op == TIS_OP_GATHER_ATTEND_DECODE || op == TIS_OP_DECODE_STEP;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  if (select) {
    p.own_scores = op != TIS_OP_TOPK_SELECT_GIVEN_SCORES;
    p.long_rows = !p.prefill_rows && n_sel_pages == 0 && p.cap > kDecodeKeyCap;
    p.pmax = !p.prefill_rows && n_sel_pages > 0 && p.own_scores;
    if (p.own_scores) p.off_scores = take((size_t)p.rows * p.cap * sizeof(float));
    if (p.pmax) p.off_pmax = take((size_t)p.rows * s->max_pages_per_seq * sizeof(float));
    if (p.long_rows) {
      p.slice_ld = (int)((p.cap + kCollectBlock - 1) / kCollectBlock);
      p.off_hist = take((size_t)p.rows * kRowHistWords * sizeof(uint32_t));
      p.off_thresh = take((size_t)p.rows * sizeof(int32_t));
      p.off_above = take((size_t)p.rows * sizeof(int32_t));
      p.off_ckey = take((size_t)p.rows * p.cap * sizeof(uint32_t));
      p.off_cpos = take((size_t)p.rows * p.cap * sizeof(int32_t));
      p.off_slice = take((size_t)p.rows * p.slice_ld * sizeof(int32_t));
    }
  }
  if (op == TIS_OP_DECODE_STEP) {
    p.own_idx = true;  // used only when the caller passes no idx
    p.off_idx = take((size_t)p.rows * topk * sizeof(int32_t));
  }
  if (op == TIS_OP_GATHER_ATTEND_DECODE || op == TIS_OP_GATHER_ATTEND_PREFILL ||
      op == TIS_OP_DECODE_STEP) {
    split_plan(s, topk, attend_decode, &p);
    p.attend_decode = attend_decode;
    if (p.n_splits > 1) {
      const size_t units = (size_t)p.rows * p.n_splits;
      // partial states per (selection row, split) of that row's query heads
      const size_t hpr = (size_t)(s->num_heads / idx_heads(s));
      p.off_po = take(units * hpr * kHeadDim * sizeof(float));
      p.off_pml = take(units * hpr * 3 * sizeof(float));
    }
  }
  p.total = off;
  return p;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(TIS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return TIS_OK;
}

// ----------------------------------------------------------- stage timing
// Opt-in: HIP events recorded on the caller's stream around every kernel
// launch, keyed by stage, read back (after the work completed) by
// tis_stage_timing_read.
enum Stage { kStClear, kStScore, kStHist, kStCollect, kStSelect, kStAttend, kStCombine,
             kStAppend, kStConvert, kNumStages };
const char* const kStageNames[kNumStages] = {"clear", "score", "hist", "collect", "select",
                                             "attend", "combine", "append", "convert"};

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  struct Rec { int stage; hipEvent_t a, b; };
  std::vector<Rec> recs;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
} g_timing;

// Runs `launch` between two recorded events when timing is on.
template <class F>
hipError_t timed(int stage, hipStream_t st, F launch) {
  if (!g_timing.on) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    a = g_timing.get();
    b = g_timing.get();
  }
  auto untimed = [&]() {  // the events go back to the pool
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (a) g_timing.pool.push_back(a);
    if (b) g_timing.pool.push_back(b);
  };
  if (!a || !b || hipEventRecord(a, st) != hipSuccess) {
    untimed();
    return launch();
  }
  hipError_t e = launch();
  if (hipEventRecord(b, st) != hipSuccess) {
    untimed();
    return e;
  }
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.recs.push_back({stage, a, b});
  return e;
}

// the selection pipeline shared by sparse_topk_select and sparse_decode_step
int run_select(const tis_shape* s, const Plan& p, const uint16_t* q_comp,
               const uint16_t* k_comp_cache, const float* scores, int64_t ld,
               const int32_t* page_table, const int32_t* seq_lens, const int32_t* q_start,
               int32_t topk, int32_t n_sel_pages, int32_t* idx, float* w, int32_t* count,
               uint64_t* page_mask, void* ws, hipStream_t st) {
  int rc;
  const float* sc = scores;
  const int hq = idx_heads(s);
  HistArgs h{};
  if (p.long_rows) {
    h.ld = p.own_scores ? p.cap : ld;
    h.seq_lens = seq_lens;
    h.q_start = q_start;
    h.rows = (int)p.rows;
    h.hq = hq;
    h.max_pages = s->max_pages_per_seq;
    h.row_hist = at<uint32_t>(ws, p.off_hist);
    h.long_row_min = kDecodeKeyCap + 1;
    // the first-digit histograms are accumulated by the scorer or by launch_hist
    rc = hip_check(timed(kStClear, st, [&] { return launch_hist_clear(h, st); }),
                   "histogram clear");
    if (rc) return rc;
  }
  if (p.own_scores) {
    float* own = at<float>(ws, p.off_scores);
    ld = p.cap;
    if (!p.prefill_rows) {
      ScoreDecodeArgs a{};
      a.q_comp = q_comp;
      a.k_comp = k_comp_cache;
      a.page_table = page_table;
      a.seq_lens = seq_lens;
      a.q_start = q_start;
      a.batch = s->batch;
      a.d_c = s->d_c;
      a.max_pages = s->max_pages_per_seq;
      a.num_phys = s->num_phys_pages;
      a.scores = own;
      a.ld = ld;
      a.hq = hq;
      a.page_max = p.pmax ? at<float>(ws, p.off_pmax) : nullptr;
      // several indexer heads: the first-digit histograms come from `hist`
      a.row_hist = p.long_rows && hq == 1 ? h.row_hist : nullptr;
      a.long_row_min = h.long_row_min;
      rc = hip_check(timed(kStScore, st, [&] { return launch_score_decode(a, st); }), "decode scorer");
    } else {
      ScorePrefillArgs a{};
      a.q_comp = q_comp;
      a.k_comp = k_comp_cache;
      a.page_table = page_table;
      a.seq_lens = seq_lens;
      a.q_start = q_start;
      a.batch = s->batch;
      a.num_q = s->num_q;
      a.d_c = s->d_c;
      a.max_pages = s->max_pages_per_seq;
      a.num_phys = s->num_phys_pages;
      a.scores = own;
      a.ld = ld;
      a.hq = hq;
      // an exact selection keeps every position of a row that sees at most
      // topk of them, reading its scores only to return them in w
      a.skip_n = w == nullptr && n_sel_pages == 0 ? topk : 0;
      rc = hip_check(timed(kStScore, st, [&] { return launch_score_prefill(a, st); }), "prefill scorer");
    }
    if (rc) return rc;
    sc = own;
  }
  if (p.long_rows) {
    if (!p.own_scores || hq > 1) {  // scores the scorer did not histogram: here
      h.scores = sc;
      rc = hip_check(timed(kStHist, st, [&] { return launch_hist(h, st); }), "histogram");
      if (rc) return rc;
    }
    CollectArgs c{};
    c.scores = sc;
    c.ld = ld;
    c.seq_lens = seq_lens;
    c.q_start = q_start;
    c.rows = (int)p.rows;
    c.hq = hq;
    c.max_pages = s->max_pages_per_seq;
    c.topk = topk;
    c.row_hist = h.row_hist;
    c.thresh = at<int32_t>(ws, p.off_thresh);
    c.above = at<int32_t>(ws, p.off_above);
    c.long_row_min = kDecodeKeyCap + 1;
    c.cand_key = at<uint32_t>(ws, p.off_ckey);
    c.cand_pos = at<int32_t>(ws, p.off_cpos);
    c.cand_ld = p.cap;
    c.slice_cnt = at<int32_t>(ws, p.off_slice);
    c.slice_ld = p.slice_ld;
    rc = hip_check(timed(kStCollect, st, [&] { return launch_collect(c, st); }), "collect");
    if (rc) return rc;
  }
  SelectArgs a{};
  a.scores = sc;
  a.ld = ld;
  a.seq_lens = seq_lens;
  a.q_start = q_start;
  a.batch = s->batch;
  a.num_q = s->num_q;
  a.hq = hq;
  a.max_pages = s->max_pages_per_seq;
  a.topk = topk;
  a.n_sel_pages = n_sel_pages;
  a.page_max = p.pmax ? at<float>(ws, p.off_pmax) : nullptr;
  if (p.long_rows) {
    a.cand_key = at<uint32_t>(ws, p.off_ckey);
    a.cand_pos = at<int32_t>(ws, p.off_cpos);
    a.slice_cnt = at<int32_t>(ws, p.off_slice);
    a.thresh = at<int32_t>(ws, p.off_thresh);
    a.above = at<int32_t>(ws, p.off_above);
    a.cand_ld = p.cap;
    a.slice_ld = p.slice_ld;
  }
  a.long_row_min = kDecodeKeyCap + 1;
  a.idx = idx;
  a.w = w;
  a.count = count;
  a.page_mask = page_mask;
  return hip_check(timed(kStSelect, st, [&] { return launch_select(a, p.prefill_rows, st); }), "select");
}

int run_attend(const tis_shape* s, const Plan& p, const uint16_t* q, const uint16_t* k_cache,
               const uint16_t* v_cache, const int32_t* page_table, const int32_t* idx,
               int32_t topk, float softmax_scale, uint16_t* out, float* lse, void* ws,
               hipStream_t st) {
  AttendArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.idx = idx;
  a.rows = (int)p.rows;  // selection rows: B * S_q * Hi
  a.num_q = s->num_q;
  a.idx_heads = idx_heads(s);
  a.num_heads = s->num_heads / a.idx_heads;  // query heads per selection row
  a.max_pages = s->max_pages_per_seq;
  a.num_phys = s->num_phys_pages;
  a.topk = topk;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)s->head_dim);
  a.keys_per_split = p.keys_per_split;
  a.n_splits = p.n_splits;
  a.out = out;
  a.lse = lse;
  a.part_o = p.n_splits > 1 ? at<float>(ws, p.off_po) : nullptr;
  a.part_ml = p.n_splits > 1 ? at<float>(ws, p.off_pml) : nullptr;
  if (!p.attend_decode && prefill_attend_supported(s->max_pages_per_seq, s->num_q, a.num_heads, topk))
    return hip_check(
        timed(kStAttend, st, [&] { return launch_prefill_attend(a, s->batch, st); }),
        "prefill attend");
  int rc = hip_check(timed(kStAttend, st, [&] { return launch_attend(a, st); }), "gather-attend");
  if (rc) return rc;
  return hip_check(timed(kStCombine, st, [&] { return launch_combine(a, st); }), "combine");
}

// ------------------------------------------------- no-allocation scratch
// The scratch memory of sparse_decode_step_noalloc: a fixed array in device
// memory, one copy per device, held from the library's load on that device
// until the process ends. Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_address(void** out) {
  int dev = -1;
  int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(TIS_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    rc = hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (rc) return rc;
    if (!ptr) return fail(TIS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TIS_OK;
}

int check_ws(const Plan& p, void* ws, size_t bytes) {
  if (bytes < p.total)
    return fail(TIS_ERR_WORKSPACE_TOO_SMALL,
                "workspace too small: need " + std::to_string(p.total) + " bytes, got " +
                    std::to_string(bytes));
  if (p.total > 0 && !ws) return fail(TIS_ERR_INVALID_ARG, "workspace is NULL");
  if (p.total > 0 && (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(TIS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return TIS_OK;
}

}  // namespace

extern "C" {

int tis_abi_version(void) { return TIS_ABI_VERSION; }

int tis_stage_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  const int prev = g_timing.on ? 1 : 0;
  g_timing.on = on != 0;
  return prev;
}

int tis_stage_timing_read(double* ms, int64_t* launches, int32_t n_stages) {
  if (!ms || !launches || n_stages < kNumStages)
    return fail(TIS_ERR_INVALID_ARG, "need arrays of at least TIS_NUM_STAGES entries");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (int i = 0; i < kNumStages; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  int rc = TIS_OK;
  for (auto& r : g_timing.recs) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) rc = hip_check(e, "stage timing");
    ms[r.stage] += t;
    launches[r.stage] += 1;
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.recs.clear();
  return rc ? rc : ok();
}

const char* tis_stage_name(int32_t stage) {
  return stage >= 0 && stage < kNumStages ? kStageNames[stage] : "";
}

const char* tis_last_error(void) { return g_error.c_str(); }

size_t tis_workspace_size(const tis_shape* shape, int32_t op, int32_t topk, int32_t n_sel_pages) {
  if (check_shape(shape)) return 0;
  if (op < TIS_OP_INDEX_SCORE || op > TIS_OP_DECODE_STEP) {
    fail(TIS_ERR_INVALID_ARG, "unknown op");
    return 0;
  }
  if (op == TIS_OP_INDEX_SCORE) return 0;
  if (check_topk(topk, op == TIS_OP_GATHER_ATTEND_DECODE || op == TIS_OP_GATHER_ATTEND_PREFILL
                           ? 0 : n_sel_pages))
    return 0;
  if (op == TIS_OP_DECODE_STEP && shape->num_q != 1) {
    fail(TIS_ERR_INVALID_ARG, "the decode step needs num_q == 1");
    return 0;
  }
  g_error.clear();
  return make_plan(shape, op, topk, n_sel_pages).total;
}

int sparse_index_score(const tis_shape* shape, const uint16_t* q_comp,
                       const uint16_t* k_comp_cache, const int32_t* page_table,
                       const int32_t* seq_lens, const int32_t* q_start, float* scores,
                       int64_t ld_scores, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q_comp || !k_comp_cache || !page_table || !scores)
    return fail(TIS_ERR_INVALID_ARG, "q_comp, k_comp_cache, page_table and scores must be set");
  if (!seq_lens && !q_start) return fail(TIS_ERR_INVALID_ARG, "need seq_lens or q_start");
  const int64_t cap = (int64_t)shape->max_pages_per_seq * kBlockSize;
  if (ld_scores < cap) return fail(TIS_ERR_INVALID_ARG, "ld_scores < max_pages_per_seq * block_size");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->num_q == 1) {
    ScoreDecodeArgs a{};
    a.q_comp = q_comp;
    a.k_comp = k_comp_cache;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.q_start = q_start;
    a.batch = shape->batch;
    a.d_c = shape->d_c;
    a.max_pages = shape->max_pages_per_seq;
    a.num_phys = shape->num_phys_pages;
    a.scores = scores;
    a.ld = ld_scores;
    a.hq = idx_heads(shape);
    rc = hip_check(timed(kStScore, st, [&] { return launch_score_decode(a, st); }), "decode scorer");
  } else {
    ScorePrefillArgs a{};
    a.q_comp = q_comp;
    a.k_comp = k_comp_cache;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.q_start = q_start;
    a.batch = shape->batch;
    a.num_q = shape->num_q;
    a.d_c = shape->d_c;
    a.max_pages = shape->max_pages_per_seq;
    a.num_phys = shape->num_phys_pages;
    a.scores = scores;
    a.ld = ld_scores;
    a.hq = idx_heads(shape);
    rc = hip_check(timed(kStScore, st, [&] { return launch_score_prefill(a, st); }), "prefill scorer");
  }
  return rc ? rc : ok();
}

int sparse_topk_select(const tis_shape* shape, const uint16_t* q_comp,
                       const uint16_t* k_comp_cache, const float* scores, int64_t ld_scores,
                       const int32_t* page_table, const int32_t* seq_lens, const int32_t* q_start,
                       int32_t topk, int32_t n_sel_pages, int32_t* idx, float* w, int32_t* count,
                       uint64_t* page_mask, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_topk(topk, n_sel_pages))) return rc;
  if (!idx) return fail(TIS_ERR_INVALID_ARG, "idx must be set");
  if (!seq_lens && !q_start) return fail(TIS_ERR_INVALID_ARG, "need seq_lens or q_start");
  const int64_t cap = (int64_t)shape->max_pages_per_seq * kBlockSize;
  if (scores) {
    if (ld_scores < cap)
      return fail(TIS_ERR_INVALID_ARG, "ld_scores < max_pages_per_seq * block_size");
  } else if (!q_comp || !k_comp_cache || !page_table) {
    return fail(TIS_ERR_INVALID_ARG, "fused scoring needs q_comp, k_comp_cache and page_table");
  }
  const Plan p = make_plan(shape, scores ? TIS_OP_TOPK_SELECT_GIVEN_SCORES : TIS_OP_TOPK_SELECT,
                           topk, n_sel_pages);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  rc = run_select(shape, p, q_comp, k_comp_cache, scores, ld_scores, page_table, seq_lens,
                  q_start, topk, n_sel_pages, idx, w, count, page_mask, workspace,
                  static_cast<hipStream_t>(stream));
  return rc ? rc : ok();
}

int paged_gather_attend(const tis_shape* shape, int32_t phase, const uint16_t* q,
                        const uint16_t* k_cache, const uint16_t* v_cache,
                        const int32_t* page_table, const int32_t* idx, int32_t topk,
                        float softmax_scale, uint16_t* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_topk(topk, 0))) return rc;
  if (phase != TIS_PHASE_DECODE && phase != TIS_PHASE_PREFILL)
    return fail(TIS_ERR_INVALID_ARG, "phase must be TIS_PHASE_DECODE or TIS_PHASE_PREFILL");
  if (!q || !k_cache || !v_cache || !page_table || !idx || !out)
    return fail(TIS_ERR_INVALID_ARG, "q, k_cache, v_cache, page_table, idx and out must be set");
  const Plan p = make_plan(shape,
                           phase == TIS_PHASE_DECODE ? TIS_OP_GATHER_ATTEND_DECODE
                                                     : TIS_OP_GATHER_ATTEND_PREFILL,
                           topk, 0);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  rc = run_attend(shape, p, q, k_cache, v_cache, page_table, idx, topk, softmax_scale, out, lse,
                  workspace, static_cast<hipStream_t>(stream));
  return rc ? rc : ok();
}

int sparse_decode_step(const tis_shape* shape, const uint16_t* q_comp,
                       const uint16_t* k_comp_cache, const uint16_t* q, const uint16_t* k_cache,
                       const uint16_t* v_cache, const int32_t* page_table,
                       const int32_t* seq_lens, int32_t topk, int32_t n_sel_pages,
                       float softmax_scale, uint16_t* out, int32_t* idx, float* w, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_topk(topk, n_sel_pages))) return rc;
  if (shape->num_q != 1) return fail(TIS_ERR_INVALID_ARG, "the decode step needs num_q == 1");
  if (!q_comp || !k_comp_cache || !q || !k_cache || !v_cache || !page_table || !seq_lens || !out)
    return fail(TIS_ERR_INVALID_ARG,
                "q_comp, k_comp_cache, q, k_cache, v_cache, page_table, seq_lens and out must be set");
  const Plan p = make_plan(shape, TIS_OP_DECODE_STEP, topk, n_sel_pages);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* sel = idx ? idx : at<int32_t>(workspace, p.off_idx);
  rc = run_select(shape, p, q_comp, k_comp_cache, nullptr, 0, page_table, seq_lens, nullptr, topk,
                  n_sel_pages, sel, w, nullptr, nullptr, workspace, st);
  if (rc) return rc;
  rc = run_attend(shape, p, q, k_cache, v_cache, page_table, sel, topk, softmax_scale, out, lse,
                  workspace, st);
  return rc ? rc : ok();
}

int sparse_decode_step_noalloc(const tis_shape* shape, const uint16_t* q_comp,
                               const uint16_t* k_comp_cache, const uint16_t* q,
                               const uint16_t* k_cache, const uint16_t* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, int32_t topk,
                               int32_t n_sel_pages, float softmax_scale, uint16_t* out,
                               int32_t* idx, float* w, float* lse, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_topk(topk, n_sel_pages))) return rc;
  if (shape->num_q != 1) return fail(TIS_ERR_INVALID_ARG, "the decode step needs num_q == 1");
  const Plan p = make_plan(shape, TIS_OP_DECODE_STEP, topk, n_sel_pages);
  if (p.total > kScratchBytes)
    return fail(TIS_ERR_UNSUPPORTED,
                "sparse_decode_step_noalloc: this shape needs " + std::to_string(p.total) +
                    " bytes of scratch memory, more than the " + std::to_string(kScratchBytes) +
                    " it holds; call sparse_decode_step with a workspace");
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return sparse_decode_step(shape, q_comp, k_comp_cache, q, k_cache, v_cache, page_table, seq_lens,
                            topk, n_sel_pages, softmax_scale, out, idx, w, lse, ws, kScratchBytes,
                            stream);
}

int mxfp4_to_fp8_experts(const uint8_t* w_packed, const uint8_t* w_scales, int32_t num_experts,
                         int32_t rows, int32_t cols, const int32_t* expert_ids, int32_t n_sel,
                         int32_t exp_offset, uint8_t* fp8_out, size_t out_bytes, void* stream) {
  if (num_experts < 1 || rows < 1 || cols < 32)
    return fail(TIS_ERR_INVALID_ARG, "num_experts and rows must be >= 1 and cols >= 32");
  if (cols % 32 != 0) return fail(TIS_ERR_UNSUPPORTED, "cols must be a multiple of 32");
  if (n_sel < 0) return fail(TIS_ERR_INVALID_ARG, "n_sel must be >= 0");
  if (n_sel > 65535) return fail(TIS_ERR_UNSUPPORTED, "n_sel must be <= 65535");
  if (exp_offset < -1024 || exp_offset > 1024)
    return fail(TIS_ERR_INVALID_ARG, "exp_offset must lie in [-1024, 1024]");
  if (n_sel == 0) return ok();
  if (!w_packed || !w_scales || !expert_ids || !fp8_out)
    return fail(TIS_ERR_INVALID_ARG, "w_packed, w_scales, expert_ids and fp8_out must be set");
  if ((reinterpret_cast<uintptr_t>(w_packed) & 7) || (reinterpret_cast<uintptr_t>(fp8_out) & 15))
    return fail(TIS_ERR_INVALID_ARG, "w_packed must be 8-byte and fp8_out 16-byte aligned");
  const int64_t per = (int64_t)rows * cols;
  if ((int64_t)num_experts * per / 2 > ((int64_t)1 << 62) / 4)
    return fail(TIS_ERR_UNSUPPORTED, "expert pool too large");
  if (out_bytes < (size_t)n_sel * (size_t)per)
    return fail(TIS_ERR_WORKSPACE_TOO_SMALL,
                "fp8_out holds " + std::to_string(out_bytes) + " bytes; n_sel * rows * cols = " +
                    std::to_string((size_t)n_sel * (size_t)per));
  Mxfp4Args a{};
  a.packed = w_packed;
  a.scales = w_scales;
  a.num_experts = num_experts;
  a.rows = rows;
  a.cols = cols;
  a.expert_ids = expert_ids;
  a.n_sel = n_sel;
  a.exp_offset = exp_offset;
  a.out = fp8_out;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rc =
      hip_check(timed(kStConvert, st, [&] { return launch_mxfp4_to_fp8(a, st); }), "mxfp4 convert");
  return rc ? rc : ok();
}

int paged_kv_append(const tis_shape* shape, const uint16_t* k_comp_new, const uint16_t* k_new,
                    const uint16_t* v_new, const int32_t* page_table, int32_t* seq_lens,
                    uint16_t* k_comp_cache, uint16_t* k_cache, uint16_t* v_cache, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!k_comp_new || !k_new || !v_new || !page_table || !seq_lens || !k_comp_cache || !k_cache ||
      !v_cache)
    return fail(TIS_ERR_INVALID_ARG, "every pointer of paged_kv_append must be set");
  AppendArgs a{};
  a.k_comp_new = k_comp_new;
  a.k_new = k_new;
  a.v_new = v_new;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.k_comp_cache = k_comp_cache;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.batch = shape->batch;
  a.d_c = shape->d_c;
  a.max_pages = shape->max_pages_per_seq;
  a.num_phys = shape->num_phys_pages;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_check(timed(kStAppend, st, [&] { return launch_append(a, st); }), "append");
  return rc ? rc : ok();
}

}  // extern "C"
