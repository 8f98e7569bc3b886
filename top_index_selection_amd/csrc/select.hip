// select.hip -- masked top-k index selection for gfx950.
//
// The top-k of each row is found by radix selection instead of a sort ("Day-0
// Inference Adaptation for Ultra-Large MoE Models on Domestic GPUs", section
// "Operatorizing Index Selection": fused top-k that avoids full sorting; "Day-0
// Inference Adaptation of Ultra-Large-Scale MoE Models on Domestic AI
// Accelerators", section 4.1: on-device top-k without element-wise sorting).
//
// Keys: each fp32 score maps to an order-preserving uint32; the selection is
// "the K' largest keys, equal keys by lower position". Digits are taken from
// the top: 12, 12 and 8 bits. Each pass histograms, in LDS, the keys that
// still match the known prefix and locates the digit of the K'-th largest.
// The result is the threshold key T and the number r of elements equal to T
// that are kept; kept = (key > T) or (key == T and among the first r such by
// position). A wave-ballot compaction in position order then writes the kept
// positions in ascending order: no sort is needed at any point.
//
// Long decode rows (more positions than fit in LDS) take a two-level path:
// `hist` builds partial histograms of the first digit per 32K-position chunk,
// `thresh` sums them and finds the digit of the K'-th largest key, `collect`
// keeps, chunk by chunk and in position order, every element whose first digit
// reaches it, and the select kernel runs the same LDS radix select over those
// candidates only. No kernel needs a device-wide fence or cross-block atomic.
//
// Block pruning ("Operatorizing Index Selection": candidates pruned at block
// granularity, then selected precisely; section 4.1: block-wise approximate
// selection followed by local exact selection) runs the same select twice:
// over the page maxima (positions = logical pages), then over the positions
// of the kept pages.
#include "tis_common.h"
#include "tis_internal.h"

namespace tis {

// ------------------------------------- first-digit histogram and threshold

// Partial histograms of the first 12-bit digit, one per 32K-position chunk of a
// long row, written with plain stores (no cross-block atomics).
__global__ __launch_bounds__(256) void hist_kernel(HistArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  const int b = blockIdx.y;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  if (rg.n < a.long_row_min) return;
  const int64_t j0 = (int64_t)blockIdx.x * kHistChunk;
  if (j0 >= rg.n) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  const float* srow = a.scores + (int64_t)b * a.ld;
  const int64_t j1 = j0 + kHistChunk < rg.n ? j0 + kHistChunk : rg.n;
  for (int64_t j = j0 + tid; j < j1; j += 256)
    atomicAdd(&s_hist[score_key(srow[j]) >> (32 - kHistBits)], 1u);
  __syncthreads();
  uint32_t* out = a.part + ((int64_t)b * a.n_chunks_ld + blockIdx.x) * kHistBins;
  for (int i = tid; i < kHistBins; i += 256) out[i] = s_hist[i];
}

hipError_t launch_hist(const HistArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(hist_kernel, dim3((unsigned)a.n_chunks_ld, (unsigned)a.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

// One block per long row: sum the partial histograms and find the digit that
// holds the K'-th largest key.
__global__ __launch_bounds__(256) void thresh_kernel(HistArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ int s_tmp[8];
  const int b = blockIdx.x;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  if (rg.n < a.long_row_min) return;
  const int nch = (int)((rg.n + kHistChunk - 1) / kHistChunk);
  const int tid = threadIdx.x;
  const uint32_t* part = a.part + (int64_t)b * a.n_chunks_ld * kHistBins;
  u32x4 acc[4] = {};
  for (int c = 0; c < nch; ++c) {
    const u32x4* src = reinterpret_cast<const u32x4*>(part + (int64_t)c * kHistBins) + tid * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += src[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(&s_hist[tid * 16 + k * 4]) = acc[k];
  __syncthreads();
  const int kk = (int)(rg.n < a.topk ? rg.n : a.topk);
  int above;
  const int d = find_digit_desc([&](int bin) { return s_hist[bin]; }, kHistBins, kk, s_tmp, &above);
  if (tid == 0) a.thresh[b] = d;
}

hipError_t launch_thresh(const HistArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(thresh_kernel, dim3((unsigned)a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------ candidate collection

// Each wave owns 256 consecutive positions and writes, in position order, the
// (key, position) of every element whose first digit is >= the threshold digit
// into its own slice of the candidate arrays, plus the slice's count.
__global__ __launch_bounds__(256) void collect_kernel(CollectArgs a) {
  const int b = blockIdx.y;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  if (rg.n < a.long_row_min) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wc = (int64_t)blockIdx.x * 4 + wave;
  const int64_t start = wc * kPositionsPerWaveChunk;
  if (start >= rg.n) return;
  const uint32_t t = (uint32_t)a.thresh[b];
  const float* srow = a.scores + (int64_t)b * a.ld;
  uint32_t* ck = a.cand_key + (int64_t)b * a.cand_ld + start;
  int32_t* cp = a.cand_pos + (int64_t)b * a.cand_ld + start;
  int running = 0;
#pragma unroll
  for (int k = 0; k < kPositionsPerWaveChunk / 64; ++k) {
    const int64_t j = start + k * 64 + lane;
    const bool in = j < rg.n;
    const uint32_t key = in ? score_key(srow[j]) : 0u;
    const bool keep = in && (key >> (32 - kHistBits)) >= t;
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int off = running + lanes_below(m);
      ck[off] = key;
      cp[off] = (int32_t)j;
    }
    running += __popcll(m);
  }
  if (lane == 0) a.wcnt[(int64_t)b * a.wcnt_ld + wc] = running;
}

hipError_t launch_collect(const CollectArgs& a, hipStream_t s) {
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int64_t blocks = (cap + 4 * kPositionsPerWaveChunk - 1) / (4 * kPositionsPerWaveChunk);
  hipLaunchKernelGGL(collect_kernel, dim3((unsigned)blocks, (unsigned)a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

// --------------------------------------------------------- per-row select

// A key source: key(e) and pos(e) for e in [0, n), in ascending position.
struct LdsKeys {
  const uint32_t* keys;
  const int32_t* pos;  // null: position = base + e
  int64_t base;
  __device__ uint32_t key(int64_t e) const { return keys[e]; }
  __device__ int64_t at(int64_t e) const { return pos ? (int64_t)pos[e] : base + e; }
};

struct GlobalScores {  // a score row in global memory, positions 0..n-1
  const float* row;
  __device__ uint32_t key(int64_t e) const { return score_key(row[e]); }
  __device__ int64_t at(int64_t e) const { return e; }
};

struct GlobalPageMax {  // page maxima in global memory, positions = pages
  const float* row;
  __device__ uint32_t key(int64_t e) const { return score_key(row[e]); }
  __device__ int64_t at(int64_t e) const { return e; }
};

struct PageMaxOfScores {  // page maxima computed from a score row on the fly
  const float* row;
  int64_t p;
  __device__ uint32_t key(int64_t g) const {
    const int64_t first = g * kBlockSize;
    const int64_t last = first + kBlockSize - 1 < p ? first + kBlockSize - 1 : p;
    float mx = row[first];
    for (int64_t j = first + 1; j <= last; ++j) mx = fmaxf(mx, row[j]);
    return score_key(mx);
  }
  __device__ int64_t at(int64_t g) const { return g; }
};

struct KeptPageScores {  // positions of the kept pages (ascending), scores in global
  const float* row;
  const int32_t* pages;
  __device__ int64_t at(int64_t e) const { return (int64_t)pages[e >> 6] * kBlockSize + (e & 63); }
  __device__ uint32_t key(int64_t e) const { return score_key(row[at(e)]); }
};

// Radix select: the K-th largest key T of src[0..n) and the number r of
// elements equal to T that belong to the top K. Requires 1 <= K <= n.
template <class Src>
__device__ void radix_select(const Src& src, int64_t n, int K, uint32_t* hist, int* tmp,
                             uint32_t* T, int* r) {
  constexpr int kShift[3] = {20, 8, 0};
  constexpr int kBits[3] = {12, 12, 8};
  uint32_t prefix = 0u, known = 0u;
  int krem = K;
  for (int pass = 0; pass < 3; ++pass) {
    const int nb = 1 << kBits[pass];
    const uint32_t dmask = (uint32_t)(nb - 1);
    for (int i = threadIdx.x; i < nb; i += 256) hist[i] = 0u;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < n; e += 256) {
      const uint32_t k = src.key(e);
      if ((k & known) == prefix) atomicAdd(&hist[(k >> kShift[pass]) & dmask], 1u);
    }
    __syncthreads();
    int above;
    const int d = find_digit_desc([&](int bin) { return hist[bin]; }, nb, krem, tmp, &above);
    krem -= above;
    prefix |= (uint32_t)d << kShift[pass];
    known |= dmask << kShift[pass];
  }
  *T = prefix;
  *r = krem;
}

// Keep (key > T) or (key == T and one of the first r such); write the kept
// positions and keys, in ascending position, to sel_pos / sel_key.
// Each wave walks a contiguous quarter of [0, n) in 64-element rounds.
template <class Src>
__device__ void ordered_compact(const Src& src, int64_t n, uint32_t T, int r, int32_t* sel_pos,
                                uint32_t* sel_key, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t quarter = ((n + 3) / 4 + 63) / 64 * 64;
  const int64_t lo = wave * quarter;
  const int64_t hi = lo + quarter < n ? lo + quarter : n;
  int gt = 0, eq = 0;
  for (int64_t e0 = lo; e0 < hi; e0 += 64) {
    const int64_t e = e0 + lane;
    const uint32_t k = e < hi ? src.key(e) : 0u;
    gt += __popcll(__ballot(e < hi && k > T));
    eq += __popcll(__ballot(e < hi && k == T));
  }
  if (lane == 0) {
    tmp[wave] = gt;
    tmp[4 + wave] = eq;
  }
  __syncthreads();
  int G = 0, E = 0;
  for (int w = 0; w < wave; ++w) {
    G += tmp[w];
    E += tmp[4 + w];
  }
  __syncthreads();
  for (int64_t e0 = lo; e0 < hi; e0 += 64) {
    const int64_t e = e0 + lane;
    const bool in = e < hi;
    const uint32_t k = in ? src.key(e) : 0u;
    const bool g = in && k > T, q = in && k == T;
    const uint64_t mg = __ballot(g), mq = __ballot(q);
    const int gb = G + lanes_below(mg), eb = E + lanes_below(mq);
    if (g || (q && eb < r)) {
      const int slot = gb + (eb < r ? eb : r);
      sel_pos[slot] = (int32_t)src.at(e);
      sel_key[slot] = k;
    }
    G += __popcll(mg);
    E += __popcll(mq);
  }
  __syncthreads();
}

// Select the top K of src[0..n) into sel_pos/sel_key (ascending position).
template <class Src>
__device__ void select_topk(const Src& src, int64_t n, int K, uint32_t* hist, int32_t* sel_pos,
                            uint32_t* sel_key, int* tmp) {
  if (K >= n) {  // everything is kept
    for (int64_t e = threadIdx.x; e < n; e += 256) {
      sel_pos[e] = (int32_t)src.at(e);
      sel_key[e] = src.key(e);
    }
    __syncthreads();
    return;
  }
  uint32_t T;
  int r;
  radix_select(src, n, K, hist, tmp, &T, &r);
  ordered_compact(src, n, T, r, sel_pos, sel_key, tmp);
}

// Row outputs from the kept list: idx (+ -1 padding), w, count, page mask.
__device__ void write_row(const SelectArgs& a, int64_t row, int K, const int32_t* sel_pos,
                          const uint32_t* sel_key) {
  const int tid = threadIdx.x;
  int32_t* idx = a.idx + row * a.topk;
  for (int e = tid; e < a.topk; e += 256) idx[e] = e < K ? sel_pos[e] : -1;
  if (a.w) {
    float* w = a.w + row * a.topk;
    for (int e = tid; e < a.topk; e += 256) w[e] = e < K ? key_score(sel_key[e]) : 0.0f;
  }
  if (a.count && tid == 0) a.count[row] = K;
  if (a.page_mask) {
    uint64_t* mrow = a.page_mask + row * a.max_pages;
    for (int g = tid; g < a.max_pages; g += 256) mrow[g] = 0ull;
    __syncthreads();
    // the first kept position of each page assembles and stores that page's word
    for (int e = tid; e < K; e += 256) {
      const int g = sel_pos[e] >> 6;
      if (e == 0 || (sel_pos[e - 1] >> 6) != g) {
        uint64_t word = 0ull;
        for (int f = e; f < K && (sel_pos[f] >> 6) == g; ++f) word |= 1ull << (sel_pos[f] & 63);
        mrow[g] = word;
      }
    }
  }
}

// Candidates of a long row, gathered from the per-wave-chunk slices into LDS
// in position order. Returns the count m, or -1 if m exceeds the capacity.
__device__ int64_t gather_candidates(const SelectArgs& a, int b, int64_t n, uint32_t* keys,
                                     int32_t* pos, int cap, int* tmp) {
  const int64_t nwc = (n + kPositionsPerWaveChunk - 1) / kPositionsPerWaveChunk;
  const int32_t* cnt = a.wcnt + (int64_t)b * a.wcnt_ld;
  // chunks handled per thread: contiguous runs so that the prefix is one scan
  const int64_t per = (nwc + 255) / 256;
  const int64_t c0 = threadIdx.x * per;
  int mine = 0;
  for (int64_t c = c0; c < c0 + per && c < nwc; ++c) mine += cnt[c];
  int total;
  const int before = block_excl_scan_256(mine, tmp, &total);
  if (total > cap) return -1;
  int off = before;
  const uint32_t* ck = a.cand_key + (int64_t)b * a.cand_ld;
  const int32_t* cp = a.cand_pos + (int64_t)b * a.cand_ld;
  for (int64_t c = c0; c < c0 + per && c < nwc; ++c) {
    const int k = cnt[c];
    const int64_t src = c * kPositionsPerWaveChunk;
    for (int e = 0; e < k; ++e) {
      keys[off + e] = ck[src + e];
      pos[off + e] = cp[src + e];
    }
    off += k;
  }
  __syncthreads();
  return total;
}

template <int KCAP, int PCAP>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  __shared__ uint32_t s_keys[KCAP];
  __shared__ int32_t s_pos[PCAP > 0 ? PCAP : 1];
  __shared__ uint32_t s_hist[kHistBins];  // radix bins, then the kept positions
  __shared__ uint32_t s_selkey[4096];
  __shared__ int32_t s_pages[256];
  __shared__ int s_tmp[16];
  int32_t* s_selpos = reinterpret_cast<int32_t*>(s_hist);

  const int64_t row = blockIdx.x;
  const int b = (int)(row / a.num_q), i = (int)(row % a.num_q);
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, a.num_q, b, i, cap);
  const int64_t n = rg.n;
  const float* srow = a.scores + row * a.ld;
  const int tid = threadIdx.x;

  if (a.n_sel_pages > 0) {
    // ---- block pruning: top pages by maximum score, then exact top-k inside
    const int64_t n_pg = (n + kBlockSize - 1) / kBlockSize;
    const int P = (int)(n_pg < a.n_sel_pages ? n_pg : a.n_sel_pages);
    if (a.page_max) {
      const float* pm = a.page_max + row * a.max_pages;
      if (n_pg <= KCAP) {
        for (int64_t g = tid; g < n_pg; g += 256) s_keys[g] = score_key(pm[g]);
        __syncthreads();
        select_topk(LdsKeys{s_keys, nullptr, 0}, n_pg, P, s_hist, s_selpos, s_selkey, s_tmp);
      } else {
        select_topk(GlobalPageMax{pm}, n_pg, P, s_hist, s_selpos, s_selkey, s_tmp);
      }
    } else if (n_pg <= KCAP) {
      // page maxima from the score row: one thread per page, over valid positions
      for (int64_t g = tid; g < n_pg; g += 256) s_keys[g] = PageMaxOfScores{srow, rg.p}.key(g);
      __syncthreads();
      select_topk(LdsKeys{s_keys, nullptr, 0}, n_pg, P, s_hist, s_selpos, s_selkey, s_tmp);
    } else {
      select_topk(PageMaxOfScores{srow, rg.p}, n_pg, P, s_hist, s_selpos, s_selkey, s_tmp);
    }
    for (int e = tid; e < P; e += 256) s_pages[e] = s_selpos[e];
    __syncthreads();
    // candidate positions of the kept pages, ascending; only the page holding
    // the query can be partial, and it is the last one in ascending order
    int64_t m = (int64_t)P * kBlockSize;
    if (P > 0 && s_pages[P - 1] == (int)(rg.p >> 6)) m -= (kBlockSize - 1) - (rg.p & 63);
    const int K = (int)(m < a.topk ? m : a.topk);
    if (PCAP > 0 && m <= PCAP && m <= KCAP) {
      for (int64_t e = tid; e < m; e += 256) {
        const int64_t j = (int64_t)s_pages[e >> 6] * kBlockSize + (e & 63);
        s_keys[e] = score_key(srow[j]);
        s_pos[e] = (int32_t)j;
      }
      __syncthreads();
      select_topk(LdsKeys{s_keys, s_pos, 0}, m, K, s_hist, s_selpos, s_selkey, s_tmp);
    } else {
      select_topk(KeptPageScores{srow, s_pages}, m, K, s_hist, s_selpos, s_selkey, s_tmp);
    }
    write_row(a, row, K, s_selpos, s_selkey);
    return;
  }

  // ---- exact top-k over every position 0..p
  const int K = (int)(n < a.topk ? n : a.topk);
  if (n <= a.topk) {
    select_topk(GlobalScores{srow}, n, K, s_hist, s_selpos, s_selkey, s_tmp);
  } else if (n <= KCAP) {
    for (int64_t e = tid; e < n; e += 256) s_keys[e] = score_key(srow[e]);
    __syncthreads();
    select_topk(LdsKeys{s_keys, nullptr, 0}, n, K, s_hist, s_selpos, s_selkey, s_tmp);
  } else {
    int64_t m = -1;
    if (PCAP > 0 && a.cand_key && n >= a.long_row_min)
      m = gather_candidates(a, b, n, s_keys, s_pos, PCAP < KCAP ? PCAP : KCAP, s_tmp);
    if (m >= K)
      select_topk(LdsKeys{s_keys, s_pos, 0}, m, K, s_hist, s_selpos, s_selkey, s_tmp);
    else
      select_topk(GlobalScores{srow}, n, K, s_hist, s_selpos, s_selkey, s_tmp);
  }
  write_row(a, row, K, s_selpos, s_selkey);
}

hipError_t launch_select(const SelectArgs& a, bool prefill_rows, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.num_q;
  if (prefill_rows)
    hipLaunchKernelGGL((select_kernel<kPrefillKeyCap, 0>), dim3((unsigned)rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((select_kernel<kDecodeKeyCap, kDecodePosCap>), dim3((unsigned)rows),
                       dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tis
