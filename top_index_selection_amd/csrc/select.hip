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
// position). An ordered compaction (wave-contiguous runs, ballot prefixes
// inside a wave, the four wave counts through LDS) then writes the kept
// positions in ascending order: no sort is needed at any point.
//
// Long decode rows (more positions than fit in LDS) take a two-level path:
// one histogram per row of the first digit (4096 bins plus 64 coarse group
// counts), built by the decode scorer as it writes the scores or, for scores
// the caller passes, by `hist` over 4096-position chunks; `collect` finds the
// digit of the K'-th largest key from it and keeps, per 4096-position slice and
// in position order, every element whose first digit reaches that digit; the
// select kernel then gathers the slices and finishes the radix select over
// those candidates only, starting at the second digit. No kernel needs a
// device-wide fence; the only cross-block atomics are the additions into the
// row histograms.
//
// Block pruning ("Operatorizing Index Selection": candidates pruned at block
// granularity, then selected precisely; section 4.1: block-wise approximate
// selection followed by local exact selection) runs the same select twice:
// over the page maxima (positions = logical pages), then over the positions
// of the kept pages.
#include <type_traits>

#include "tis_common.h"
#include "tis_internal.h"

namespace tis {

// LDS scratch of a selection block of NT threads, in ints: the block scan's
// wave partials, the digit search's result, a flag, and the compaction's
// per-wave counts.
template <int NT>
struct SelTmp {
  static constexpr int kWaves = NT / kWave;
  static constexpr int kDigit = kWaves;           // 3 ints: digit, count above, count in bin
  static constexpr int kFlag = kWaves + 3;
  static constexpr int kGreater = kWaves + 4;     // kWaves ints
  static constexpr int kEqual = 2 * kWaves + 4;   // kWaves ints
  static constexpr int kSize = 3 * kWaves + 4;
};

// Among the NB radix bins, scanned from the highest digit down, find the bin d
// that holds the krem-th largest element: the count above d is < krem and the
// count above d plus count[d] is >= krem. Returns d and stores the count above
// it in *above and the count of bin d in *count. Each owning thread holds BPT
// consecutive bins (BPT = NB / NT, at least 1; with fewer bins than threads
// only the first NB threads own one): thread t the BPT bins just below
// NB - BPT * t. Requires 1 <= krem <= total count. NT threads; contains
// __syncthreads().
template <int NT, int NB, class Get>
__device__ __forceinline__ int find_digit(Get get, int krem, int* tmp, int* above, int* count) {
  constexpr int BPT = NB >= NT ? NB / NT : 1;
  constexpr int OWNERS = NB / BPT;
  using T = SelTmp<NT>;
  const int t = threadIdx.x;
  const bool own = OWNERS == NT || t < OWNERS;
  const int hi = NB - 1 - t * BPT;
  // the sum is order-free: lanes start at different bins of their runs, so
  // that one read instruction of the wave touches many LDS banks
  int sum = 0;
  if (own) {
#pragma unroll
    for (int e = 0; e < BPT; ++e) sum += (int)get(hi - ((e + t) & (BPT - 1)));
  }
  int total;
  const int excl = block_excl_scan<NT>(sum, tmp, &total);
  if (own && excl < krem && krem <= excl + sum) {  // one thread: its run, in order
    int c[BPT];
#pragma unroll
    for (int e = 0; e < BPT; ++e) c[e] = (int)get(hi - e);
    // (the bin's own count is kept as it is found: indexing c[] with a run-time
    // value would place the array in scratch memory)
    int cum = excl, found = -1, before = excl, in_found = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      if (found < 0 && cum + c[e] >= krem) {
        found = e;
        before = cum;
        in_found = c[e];
      }
      cum += c[e];
    }
    tmp[T::kDigit] = hi - found;
    tmp[T::kDigit + 1] = before;
    tmp[T::kDigit + 2] = in_found;
  }
  __syncthreads();
  const int d = tmp[T::kDigit];
  *above = tmp[T::kDigit + 1];
  *count = tmp[T::kDigit + 2];
  __syncthreads();
  return d;
}

// ------------------------------------------------------- first-digit histogram

// Zeroes the per-row histograms (fine bins and coarse counts) before the
// decode scorer or `hist` adds into them: one block per row, 16-byte stores.
__global__ __launch_bounds__(256) void hist_clear_kernel(HistArgs a) {
  u32x4* h = reinterpret_cast<u32x4*>(a.row_hist + (int64_t)blockIdx.x * kRowHistWords);
  for (int i = threadIdx.x; i < kRowHistWords / 4; i += 256) h[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_hist_clear(const HistArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(hist_clear_kernel, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

// One block of kHistThreads threads per kHistChunk-position chunk of a long
// row: an LDS histogram of the first 12-bit digit, whose nonzero bins are then
// added into the row's histogram (large chunks and blocks: each flush of the
// 4096 bins serves more positions and is spread over more waves). The loads of
// a thread are all issued before the first is used.
__global__ __launch_bounds__(kHistThreads) void hist_kernel(HistArgs a) {
  constexpr int NT = kHistThreads;
  __shared__ uint32_t s_hist[kHistBins];
  const int row = blockIdx.y, b = row / a.hq;  // decode: one query row per sequence
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  if (rg.n < a.long_row_min) return;
  const int64_t j0 = (int64_t)blockIdx.x * kHistChunk;
  if (j0 >= rg.n) return;
  const int tid = threadIdx.x;
  constexpr int U = kHistChunk / NT;
  const float* srow = a.scores + (int64_t)row * a.ld;
  float v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = j0 + u * NT + tid;
    v[u] = j < rg.n ? srow[j] : 0.0f;
  }
  for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (j0 + u * NT + tid < rg.n) atomicAdd(&s_hist[score_key(v[u]) >> (32 - kHistBits)], 1u);
  __syncthreads();
  add_row_hist<NT>(s_hist, a.row_hist + (int64_t)row * kRowHistWords);
}

hipError_t launch_hist(const HistArgs& a, hipStream_t s) {
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int64_t chunks = (cap + kHistChunk - 1) / kHistChunk;
  hipLaunchKernelGGL(hist_kernel, dim3((unsigned)chunks, (unsigned)a.rows), dim3(kHistThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------ candidate collection

// One block per 4096-position slice of a long row. The block loads its scores
// (all in flight at once) while it finds the threshold digit from
// the row's coarse and fine histograms; it then keeps, in position order, the
// (key, position) of every score whose first digit reaches the threshold
// digit: each wave counts its kept elements, the counts meet in LDS, and each
// wave writes its run at its offset within the slice. NT threads: 256 when the
// launch has blocks to spare (several per CU), 1024 when it has at most one
// block per CU (a few very long rows), so that those few blocks hold more waves.
template <int NT>
__global__ __launch_bounds__(NT) void collect_kernel(CollectArgs a) {
  constexpr int NW = NT / 64;
  __shared__ int s_cnt[NW];
  constexpr int R = kCollectBlock / NT;  // 64-position rounds per wave
  const int row = blockIdx.y, b = row / a.hq;  // decode: one query row per sequence
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the coarse counts do not depend on the row length: their read is issued
  // first, beside the one of the length
  const uint32_t* rh = a.row_hist + (int64_t)row * kRowHistWords;
  const int gc = (int)rh[kHistBins + (kHistGroups - 1 - lane)];
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  if (rg.n < a.long_row_min) return;
  const int64_t j0 = (int64_t)blockIdx.x * kCollectBlock;
  if (j0 >= rg.n) return;
  const int64_t jw = j0 + (int64_t)wave * (kCollectBlock / NW);
  const float* srow = a.scores + (int64_t)row * a.ld;
  float v[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t j = jw + k * 64 + lane;
    v[k] = j < rg.n ? srow[j] : 0.0f;
  }
  // The digit t of the K'-th largest key, found by every wave on its own:
  // lane l takes coarse group 63 - l (descending), a wave prefix sum gives the
  // keys in the groups at or above it, and the first lane to reach K' names the
  // group; the same over that group's 64 fine bins names the digit.
  // (K' is topk itself: these rows are longer than any topk, which the
  // launcher checks, so the search does not wait for the row length)
  const int kk = a.topk;
  const int gi = wave_incl_scan(gc);
  const uint64_t greach = __ballot(gi >= kk);
  const int gl = greach ? __builtin_ctzll(greach) : 63;  // wave-uniform
  const int grp = kHistGroups - 1 - gl;
  const int in_groups_above = __builtin_amdgcn_readlane(gi, gl) - __builtin_amdgcn_readlane(gc, gl);
  const int fc = (int)rh[grp * 64 + (63 - lane)];
  const int fi = wave_incl_scan(fc) + in_groups_above;
  const uint64_t freach = __ballot(fi >= kk);
  const int fl = freach ? __builtin_ctzll(freach) : 63;
  const uint32_t t = (uint32_t)(grp * 64 + 63 - fl);
  if (blockIdx.x == 0 && tid == 0) {
    a.thresh[row] = (int32_t)t;
    a.above[row] = __builtin_amdgcn_readlane(fi, fl) - __builtin_amdgcn_readlane(fc, fl);
  }
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t j = jw + k * 64 + lane;
    cnt += __popcll(__ballot(j < rg.n && (score_key(v[k]) >> (32 - kHistBits)) >= t));
  }
  if (lane == 0) s_cnt[wave] = cnt;
  __syncthreads();
  int run = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    run += w < wave ? s_cnt[w] : 0;
    total += s_cnt[w];
  }
  uint32_t* ck = a.cand_key + (int64_t)row * a.cand_ld + j0;
  int32_t* cp = a.cand_pos + (int64_t)row * a.cand_ld + j0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t j = jw + k * 64 + lane;
    const uint32_t key = score_key(v[k]);
    const bool keep = j < rg.n && (key >> (32 - kHistBits)) >= t;
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int off = run + lanes_below(m);
      ck[off] = key;
      cp[off] = (int32_t)j;
    }
    run += __popcll(m);
  }
  if (tid == 0) a.slice_cnt[(int64_t)row * a.slice_ld + blockIdx.x] = total;
}

hipError_t launch_collect(const CollectArgs& a, hipStream_t s) {
  if (a.long_row_min <= a.topk) return hipErrorInvalidValue;  // K' = topk on every long row
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int64_t blocks = (cap + kCollectBlock - 1) / kCollectBlock;
  const dim3 grid((unsigned)blocks, (unsigned)a.rows);
  if (blocks * a.rows <= device_cus()) hipLaunchKernelGGL(collect_kernel<1024>, grid, dim3(1024), 0, s, a);
  else hipLaunchKernelGGL(collect_kernel<256>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// --------------------------------------------------------- per-row select

// A key source: key(e) and pos(e) for e in [0, n), in ascending position.
struct LdsKeys {
  const uint32_t* keys;
  const int32_t* pos;  // null: position = base + e
  int base;
  __device__ uint32_t key(int e) const { return keys[e]; }
  __device__ int at(int e) const { return pos ? pos[e] : base + e; }
};

struct GlobalScores {  // a score row in global memory, positions 0..n-1
  const float* row;
  __device__ uint32_t key(int e) const { return score_key(row[e]); }
  __device__ int at(int e) const { return e; }
};

struct GlobalPageMax {  // page maxima in global memory, positions = pages
  const float* row;
  __device__ uint32_t key(int e) const { return score_key(row[e]); }
  __device__ int at(int e) const { return e; }
};

struct PageMaxOfScores {  // page maxima computed from a score row on the fly
  const float* row;
  int p;
  __device__ __forceinline__ uint32_t key(int g) const {
    const int first = g * kBlockSize;
    const int last = first + kBlockSize - 1 < p ? first + kBlockSize - 1 : p;
    float mx = -INFINITY;
    for (int j0 = first; j0 <= last; j0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = j0 + u <= last ? row[j0 + u] : -INFINITY;
#pragma unroll
      for (int u = 0; u < 8; ++u) mx = fmaxf(mx, v[u]);
    }
    return score_key(mx);
  }
  __device__ int at(int g) const { return g; }
};

struct KeptPageScores {  // positions of the kept pages (ascending), scores in global
  const float* row;
  const int32_t* pages;
  __device__ int at(int e) const { return pages[e >> 6] * kBlockSize + (e & 63); }
  __device__ uint32_t key(int e) const { return score_key(row[at(e)]); }
};

// Calls f(e, key(e)) for e = threadIdx.x, threadIdx.x + NT, ... < n. Keys are
// fetched U at a time before any is used. The selection runs as one block, so
// its cost is latency, including fetching its own instructions: unrolled loops
// are kept for the global reads that fill LDS, and the rest stay rolled.
template <int NT, int U = 1, class Src, class F>
__device__ __forceinline__ void for_keys(const Src& src, int n, F f) {
  const int t = threadIdx.x;
  int b0 = 0;
  // whole rounds: every element in range, so no per-element bound test or
  // clamp (every read is issued before any is used, so none waits for the
  // others)
  for (; b0 + NT * U <= n; b0 += NT * U) {
    uint32_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) k[u] = src.key(b0 + u * NT + t);
#pragma unroll
    for (int u = 0; u < U; ++u) f(b0 + u * NT + t, k[u]);
  }
  if (b0 < n) {  // the last, partial round (block-uniform test)
    uint32_t k[U];
    // reads past the end take the last element again
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = b0 + u * NT + t;
      k[u] = src.key(e < n ? e : n - 1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = b0 + u * NT + t;
      if (e < n) f(e, k[u]);
    }
  }
}

// Keys fetched per thread and round: rounds of 1024 keys in the radix passes,
// 4096 in the fills that stage keys into LDS.
template <int NT> constexpr int kPassU = 1024 / NT > 0 ? 1024 / NT : 1;
template <int NT> constexpr int kFillU = 4096 / NT;

// Radix select over src[0..n): the K-th largest key T and the number r of
// elements equal to T that belong to the top K. The passes start at
// `first_pass` with the digits above it already fixed: `prefix` holds them,
// `known` masks them, and krem counts what is still to be taken among the
// elements that match the prefix (1 <= krem <= their number). With hist0 the
// caller has already built the histogram of the first pass in `hist`.
template <int NT, class Src>
__device__ __forceinline__ void radix_select(const Src& src, int n, int first_pass, uint32_t prefix,
                             uint32_t known, int krem, uint32_t* hist, int* tmp, uint32_t* T,
                             int* r, bool hist0 = false) {
#pragma unroll 1
  for (int pass = first_pass; pass < 3; ++pass) {
    const int nb = pass < 2 ? 4096 : 256;
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const uint32_t dmask = (uint32_t)(nb - 1);
    if (!(hist0 && pass == first_pass)) {
      for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0u;
      __syncthreads();
      for_keys<NT, kPassU<NT>>(src, n, [&](int, uint32_t k) {
        if ((k & known) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
      });
      __syncthreads();
    }
    int above, in_bin;
    const int d = pass < 2
        ? find_digit<NT, 4096>([&](int bin) { return hist[bin]; }, krem, tmp, &above, &in_bin)
        : find_digit<NT, 256>([&](int bin) { return hist[bin]; }, krem, tmp, &above, &in_bin);
    krem -= above;
    prefix |= (uint32_t)d << shift;
    known |= dmask << shift;
    if (in_bin == krem && pass < 2) {
      // the whole bin is kept, so the selection is every key >= the bin's
      // smallest key: T just below it and no equal keys to ration (with the
      // lowest possible prefix every key is kept)
      *T = prefix ? prefix - 1u : 0u;
      *r = prefix ? 0 : INT32_MAX;
      return;
    }
  }
  *T = prefix;
  *r = krem;
}

// Keep (key > T) or (key == T and one of the first r such); write the kept
// positions, in ascending position, to sel_pos, their keys to sel_key unless it
// is null, and their scores straight to the row's global w_out unless that is
// null. Rounds of 4096 elements: each of the block's NW waves takes 4096 / NW
// consecutive elements of the round, 64 at a time, lane l element 64u + l, so
// that every key read touches consecutive words. The wave counts its (key >
// T) and (key == T) elements, the wave counts meet in LDS, and the kept slot of
// an element is then (# greater before it) + min(# equal before it, r), with
// "before it" inside the wave from ballots over the lower lanes. (Counting
// with bit counts of ballots instead of a lane scan was slower: the ballots
// then stay in scalar registers across the barrier, and those spill.)
template <int NT, bool WHOLE_ROUNDS = false, class Src>
__device__ __forceinline__ void ordered_compact(const Src& src, int n, uint32_t T, int r, int32_t* sel_pos,
                                uint32_t* sel_key, float* w_out, int* tmp) {
  constexpr int NW = NT / 64;
  constexpr int R = 64 / NW;       // 64-element steps per wave and round
  constexpr int RB = NW * 64 * R;  // elements per round: 4096
  using TT = SelTmp<NT>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // With WHOLE_ROUNDS a round is compiled twice, and whole rounds (every
  // element in range) test no element against n: fewer instructions per
  // element, more code (which only the short-row kernel takes).
  if (r == 0 || r == INT32_MAX) {
    // No equal key is rationed (the radix select stopped at a bin kept whole):
    // one predicate, key > T, or every key when r says so (T is then 0).
    const bool every = r != 0;
    int G = 0;
    auto round = [&](int r0, auto whole) {
      constexpr bool W = decltype(whole)::value;
      const int w0 = r0 + wave * 64 * R;
      uint32_t k[R];
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int e = w0 + 64 * u + lane;
        k[u] = src.key(W || e < n ? e : n - 1);
      }
      int c = 0;
#pragma unroll
      for (int u = 0; u < R; ++u) c += ((W || w0 + 64 * u + lane < n) && (every || k[u] > T)) ? 1 : 0;
      c = wave_incl_scan(c);
      if (lane == 63) tmp[TT::kGreater + wave] = c;
      __syncthreads();
      int gb = G, tg = 0;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const int cg = tmp[TT::kGreater + v];
        gb += v < wave ? cg : 0;
        tg += cg;
      }
      __syncthreads();  // the counts are read before the next round writes them
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int e = w0 + 64 * u + lane;
        const bool g = (W || e < n) && (every || k[u] > T);
        const uint64_t mg = __ballot(g);
        if (g) {
          const int slot = gb + lanes_below(mg);
          sel_pos[slot] = src.at(e);
          if (sel_key) sel_key[slot] = k[u];
          if (w_out) w_out[slot] = key_score(k[u]);
        }
        gb += __popcll(mg);
      }
      G += tg;
    };
    for (int r0 = 0; r0 < n; r0 += RB) {
      if (WHOLE_ROUNDS && r0 + RB <= n) round(r0, std::true_type{});
      else round(r0, std::false_type{});
    }
    __syncthreads();
    return;
  }
  int G = 0, Q = 0;  // block-uniform totals of the rounds before
  auto round = [&](int r0, auto whole) {
    constexpr bool W = decltype(whole)::value;
    const int w0 = r0 + wave * 64 * R;
    uint32_t k[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int e = w0 + 64 * u + lane;
      k[u] = src.key(W || e < n ? e : n - 1);
    }
    // per-lane (greater, equal) counts packed in one word, summed over the wave
    int c = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const bool in = W || w0 + 64 * u + lane < n;
      c += (in && k[u] > T) ? (1 << 16) : 0;
      c += (in && k[u] == T) ? 1 : 0;
    }
    c = wave_incl_scan(c);
    if (lane == 63) {
      tmp[TT::kGreater + wave] = c >> 16;
      tmp[TT::kEqual + wave] = c & 0xffff;
    }
    __syncthreads();
    int gb = G, eb = Q, tg = 0, tq = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int cg = tmp[TT::kGreater + v], cq = tmp[TT::kEqual + v];
      gb += v < wave ? cg : 0;
      eb += v < wave ? cq : 0;
      tg += cg;
      tq += cq;
    }
    __syncthreads();  // the counts are read before the next round writes them
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int e = w0 + 64 * u + lane;
      const bool in = W || e < n;
      const bool g = in && k[u] > T, q = in && k[u] == T;
      const uint64_t mg = __ballot(g), mq = __ballot(q);
      const int gi = gb + lanes_below(mg), qi = eb + lanes_below(mq);
      if (g || (q && qi < r)) {
        const int slot = gi + (qi < r ? qi : r);
        sel_pos[slot] = src.at(e);
        if (sel_key) sel_key[slot] = k[u];
        if (w_out) w_out[slot] = key_score(k[u]);
      }
      gb += __popcll(mg);
      eb += __popcll(mq);
    }
    G += tg;
    Q += tq;
  };
  for (int r0 = 0; r0 < n; r0 += RB) {
    if (WHOLE_ROUNDS && r0 + RB <= n) round(r0, std::true_type{});
    else round(r0, std::false_type{});
  }
  __syncthreads();
}

// Keep every element of src[0..n): positions to sel_pos, keys to sel_key and
// scores to the row's global w_out (each unless null).
template <int NT, class Src>
__device__ __forceinline__ void keep_all(const Src& src, int n, int32_t* sel_pos, uint32_t* sel_key,
                                         float* w_out) {
  if (!sel_key && !w_out) {  // positions only: no key is read
    for (int e = threadIdx.x; e < n; e += NT) sel_pos[e] = src.at(e);
    __syncthreads();
    return;
  }
  for_keys<NT, 2048 / NT>(src, n, [&](int e, uint32_t k) {
    sel_pos[e] = src.at(e);
    if (sel_key) sel_key[e] = k;
    if (w_out) w_out[e] = key_score(k);
  });
  __syncthreads();
}

// Select the top K of src[0..n) into sel_pos (ascending position) and, unless
// it is null, their keys into sel_key, and unless it is null, their scores into
// the row's global w_out.
template <int NT, bool WHOLE_ROUNDS = false, class Src>
__device__ __forceinline__ void select_topk(const Src& src, int n, int K, uint32_t* hist, int32_t* sel_pos,
                            uint32_t* sel_key, float* w_out, int* tmp, bool hist0 = false) {
  if (K >= n) {  // everything is kept
    keep_all<NT>(src, n, sel_pos, sel_key, w_out);
    return;
  }
  uint32_t T;
  int r;
  radix_select<NT>(src, n, 0, 0u, 0u, K, hist, tmp, &T, &r, hist0);
  ordered_compact<NT, WHOLE_ROUNDS>(src, n, T, r, sel_pos, sel_key, w_out, tmp);
}

// Row outputs from the kept list: idx (+ -1 padding), w (the kept keys turned
// back into scores, or, without sel_key, the scores read back from the score
// row; with w_done the selection wrote the kept scores and only the padding is
// left), count, page mask. With `direct` the selection wrote the K kept entries
// of idx and w itself (there is then no page mask), and only the padding and
// the count are left.
template <int NT>
__device__ __forceinline__ void write_row(const SelectArgs& a, int64_t row, int K, const int32_t* sel_pos,
                          const uint32_t* sel_key, const float* srow, bool w_done,
                          bool direct = false) {
  const int tid = threadIdx.x;
  int32_t* idx = a.idx + row * a.topk;
  float* w = a.w ? a.w + row * a.topk : nullptr;
  if (direct) {
    for (int e = K + tid; e < a.topk; e += NT) {
      idx[e] = -1;
      if (w) w[e] = 0.0f;
    }
    if (a.count && tid == 0) a.count[row] = K;
    return;
  }
  if (w && sel_key && !w_done) {
    // idx and w together, four entries per thread and round: every LDS read
    // of a round is issued before its global stores
    constexpr int U = 4;
    for (int e0 = tid; e0 < a.topk; e0 += NT * U) {
      int p[U];
      uint32_t k[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + NT * u;
        const bool kept = e < K;
        p[u] = kept ? sel_pos[e] : -1;
        k[u] = kept ? sel_key[e] : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + NT * u;
        if (e < a.topk) {
          idx[e] = p[u];
          w[e] = e < K ? key_score(k[u]) : 0.0f;
        }
      }
    }
  } else {
    for (int e = tid; e < a.topk; e += NT) idx[e] = e < K ? sel_pos[e] : -1;
    if (w) {
      for (int e = (w_done ? K : 0) + tid; e < a.topk; e += NT)
        w[e] = e < K ? (sel_key ? key_score(sel_key[e]) : srow[sel_pos[e]]) : 0.0f;
    }
  }
  if (a.count && tid == 0) a.count[row] = K;
  if (a.page_mask) {
    uint64_t* mrow = a.page_mask + row * a.max_pages;
    for (int g = tid; g < a.max_pages; g += NT) mrow[g] = 0ull;
    __syncthreads();  // the zeros are in place before any OR below
    // thread t takes the kept entries 8t..8t+7 of each 8·NT-entry round; they are
    // ascending, so it ORs their bits into one word per page it touches and
    // flushes each word with one atomic OR (a page's entries may span threads)
    constexpr int E = 8;
    for (int e0 = tid * E; e0 < K; e0 += NT * E) {
      int cur = -1;
      uint64_t word = 0ull;
#pragma unroll
      for (int u = 0; u < E; ++u) {
        if (e0 + u >= K) break;
        const int p = sel_pos[e0 + u];
        if ((p >> 6) != cur) {
          if (cur >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&mrow[cur]), word);
          cur = p >> 6;
          word = 0ull;
        }
        word |= 1ull << (p & 63);
      }
      if (cur >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&mrow[cur]), word);
    }
  }
}

// Candidates of a long row, gathered from its collect slices into LDS in
// position order. Returns the count m, or -1 if m exceeds the capacity. The
// exclusive prefix of the slice counts goes to `off` (LDS); thread t then
// copies the 8 consecutive output slots 8t..8t+7 of each 8·NT-slot round, two
// rounds at a time: a branchless binary search (fixed depth) finds the slice
// of a group's first slot, and the rest follow by stepping to the next slice
// when one is exhausted.
template <int NT>
__device__ __forceinline__ int gather_candidates(const SelectArgs& a, int64_t row, int n,
                                                 uint32_t* keys, int32_t* pos, int cap, int* off,
                                                 int* tmp) {
  const int ns = (int)((n + kCollectBlock - 1) / kCollectBlock);
  if (ns > kHistBins) return -1;  // more slices than `off` holds: use the fallback
  constexpr int U = kHistBins / NT;
  const int32_t* cnt = a.slice_cnt + row * a.slice_ld;
  const uint32_t* ck = a.cand_key + row * a.cand_ld;
  const int32_t* cp = a.cand_pos + row * a.cand_ld;
  const int tid = threadIdx.x;
  int c[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int q = tid * U + u;
    c[u] = q < ns ? cnt[q] : 0;
  }
  int mine = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) mine += c[u];
  int total;
  int run = block_excl_scan<NT>(mine, tmp, &total);
  if (total > cap) return -1;  // block-uniform
#pragma unroll
  for (int u = 0; u < U; ++u) {
    off[tid * U + u] = run;
    run += c[u];
  }
  __syncthreads();
  // Two groups of S slots per thread and pass (slots 8t.. of two 8·NT-slot
  // rounds): each group finds its slice on its own, and the loads of both are
  // in flight before any is stored, so 16·NT candidates cost one round trip.
  constexpr int S = 8, GR = 2;
  for (int i00 = tid * S; i00 < total; i00 += GR * NT * S) {
    uint32_t kv[GR][S];
    int32_t pv[GR][S];
#pragma unroll
    for (int gi = 0; gi < GR; ++gi) {
      const int i0 = i00 + gi * NT * S;
      // the last slice q < ns with off[q] <= i0 (slices of equal offset are
      // empty except the last of them)
      int q = 0;
#pragma unroll
      for (int step = kHistBins / 2; step >= 1; step >>= 1)
        if (q + step < ns && off[q + step] <= i0) q += step;
      int end = q + 1 < ns ? off[q + 1] : total;
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int i = i0 + u;
        kv[gi][u] = 0u;
        pv[gi][u] = 0;
        if (i < total) {
          while (i >= end) {  // step over exhausted (and empty) slices
            ++q;
            end = q + 1 < ns ? off[q + 1] : total;
          }
          const int64_t src = (int64_t)q * kCollectBlock + (i - off[q]);
          kv[gi][u] = ck[src];
          pv[gi][u] = cp[src];
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < GR; ++gi)
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int i = i00 + gi * NT * S + u;
        if (i < total) {
          keys[i] = kv[gi][u];
          pos[i] = pv[gi][u];
        }
      }
  }
  __syncthreads();
  return total;
}

// The same gather with the candidate loads issued together with the slice
// counts, before the counts are known: the NT threads split into teams of T =
// NT / (slices rounded up to a power of two), team q takes slice q, and its
// thread j loads the slice's candidates j, j + T, ... (S per thread: a budget
// of T*S per slice). Once the counts are scanned, each thread writes the loaded
// candidates that exist to their place. Returns the count m, -1 if it exceeds
// the capacity, or -2 if some slice holds more candidates than its budget or
// there are more than 32 slices (the caller then gathers the row the
// two-round way).
template <int NT>
__device__ __forceinline__ int gather_candidates_spec(const SelectArgs& a, int64_t row, int n,
                                                      uint32_t* keys, int32_t* pos, int cap,
                                                      int* tmp) {
  const int ns = (int)((n + kCollectBlock - 1) / kCollectBlock);
  // teams of at least 8 threads, whose loads cover consecutive candidates
  // (with more slices, lanes would each read a different slice)
  if (ns > 32) return -2;  // block-uniform
  int np2 = 1;
  while (np2 < ns) np2 <<= 1;
  const int T = NT / np2;  // threads per slice (block-uniform)
  constexpr int S = 24 * 256 / NT;
  const int tid = threadIdx.x, q = tid / T, j = tid - q * T;
  const bool team = q < ns;
  const int32_t* cnt = a.slice_cnt + row * a.slice_ld;
  const uint32_t* ck = a.cand_key + row * a.cand_ld + (int64_t)(team ? q : 0) * kCollectBlock;
  const int32_t* cp = a.cand_pos + row * a.cand_ld + (int64_t)(team ? q : 0) * kCollectBlock;
  const int c = team ? cnt[q] : 0;
  // a slice holds at most as many candidates as positions: reads stay below
  // that bound (inside the row's region of the candidate arrays)
  const int lim = team ? min(kCollectBlock, n - q * kCollectBlock) : 1;
  uint32_t kv[S];
  int32_t pv[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int i = j + T * s;
    const int ii = i < lim ? i : 0;
    kv[s] = ck[ii];
    pv[s] = cp[ii];
  }
  const bool over = c > T * S;
  const int mine = (team && j == 0) ? c : 0;
  int total;
  const int excl = block_excl_scan<NT>(mine, tmp, &total);
  const int base = excl - (j > 0 ? c : 0);  // the team leader's prefix
  // any slice over budget: every thread learns it through LDS
  constexpr int kFlag = SelTmp<NT>::kFlag;
  if (tid == 0) tmp[kFlag] = 0;
  __syncthreads();
  if (over) tmp[kFlag] = 1;
  __syncthreads();
  const bool any_over = tmp[kFlag] != 0;
  __syncthreads();  // the flag is read before the callee reuses tmp
  if (any_over) return -2;
  if (total > cap) return -1;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int i = j + T * s;
    if (team && i < c) {
      keys[base + i] = kv[s];
      pos[base + i] = pv[s];
    }
  }
  __syncthreads();
  return total;
}

// The same gather for rows of many short slices (the candidates of a very long
// row spread thinly over its slices): wave w takes slices w, w + NW, ..., at
// most P of them, and lane l loads candidate l of each, all issued with the
// slice counts and before any is used (a budget of 64 per slice: one coalesced
// load per slice and array). Once the counts are scanned, each lane writes its
// candidates that exist to their place. Returns the count m, -1 if it exceeds
// the capacity, or -2 if some slice holds more than 64 candidates or the row
// has more than NW * P slices.
template <int NT>
__device__ __forceinline__ int gather_candidates_wave(const SelectArgs& a, int64_t row, int n,
                                                      uint32_t* keys, int32_t* pos, int cap,
                                                      int* off, int* tmp) {
  constexpr int NW = NT / 64, P = 16;
  const int ns = (int)((n + kCollectBlock - 1) / kCollectBlock);
  if (ns > NW * P) return -2;  // block-uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* cnt = a.slice_cnt + row * a.slice_ld;
  const uint32_t* ck = a.cand_key + row * a.cand_ld;
  const int32_t* cp = a.cand_pos + row * a.cand_ld;
  int c[P];
  uint32_t kv[P];
  int32_t pv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int q = wave + NW * p;
    c[p] = 0;
    kv[p] = 0u;
    pv[p] = 0;
    if (q < ns) {  // wave-uniform
      c[p] = cnt[q];
      // a slice holds at most as many candidates as positions: reads stay
      // below that bound (inside the row's region of the candidate arrays)
      const int lim = min(kCollectBlock, n - q * kCollectBlock);
      const int64_t src = (int64_t)q * kCollectBlock + (lane < lim ? lane : 0);
      kv[p] = ck[src];
      pv[p] = cp[src];
    }
  }
  // the counts in slice order, then their exclusive prefix (one slice per
  // thread: ns <= NW * P <= NT)
  constexpr int kFlag = SelTmp<NT>::kFlag;
  if (tid == 0) tmp[kFlag] = 0;
  bool over = false;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int q = wave + NW * p;
    over |= c[p] > 64;
    if (lane == 0 && q < ns) off[q] = c[p];
  }
  __syncthreads();
  if (over) tmp[kFlag] = 1;
  const int mine = tid < ns ? off[tid] : 0;
  int total;
  const int excl = block_excl_scan<NT>(mine, tmp, &total);  // (its barriers order the flag)
  const bool any_over = tmp[kFlag] != 0;
  if (tid < ns) off[tid] = excl;
  __syncthreads();
  if (any_over) return -2;
  if (total > cap) return -1;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int q = wave + NW * p;
    if (q < ns && lane < c[p]) {
      const int at = off[q] + lane;
      keys[at] = kv[p];
      pos[at] = pv[p];
    }
  }
  __syncthreads();
  return total;
}

// Prefill rows (KCAP 8192, no position buffer): many blocks of 512 threads and
// 49 KiB of LDS, three of which fit a CU when the registers allow six waves
// per SIMD, which the launch bound asks for. Decode rows: few blocks, each
// holding the large LDS key and position buffers, so one block per CU; such a
// block has 1024 threads (four waves per SIMD), so that the latency of each
// LDS pass and of each round of global reads is spread over four times the
// waves (rounds of keys and compactions of 4096 elements either way).
// FULL = false is the short-row kernel: exact top-k only (no block pruning),
// and the launcher guarantees that every row fits in LDS (n <= KCAP), so the
// other paths are compiled out and the kernel's code is a fraction of the
// size (a selection block runs alone on its row and also waits on its own
// instruction fetches).
// DIRECT (no page mask asked for): the final selection writes the kept
// positions and scores straight to the row's idx and w, its slots being their
// final places; otherwise they go through LDS. The choice is made at launch,
// so that each instantiation stores to one address space (a destination chosen
// at run time would make every store a generic one).
// MANY_SLICES (tables wider than 32 candidate slices): long rows of more than
// 32 slices gather their candidates a wave per slice; the other instantiations
// leave that path out, so that their code and registers stay as they are.
template <int KCAP, int PCAP, bool FULL, bool DIRECT, int NT, bool MANY_SLICES = false>
__global__ __launch_bounds__(NT, PCAP > 0 ? 1 : 3) void select_kernel(SelectArgs a) {
  __shared__ uint32_t s_keys[KCAP];
  __shared__ int32_t s_pos[PCAP > 0 ? PCAP : 1];
  __shared__ uint32_t s_hist[kHistBins];  // radix bins, then the kept positions
  __shared__ int32_t s_pages[256];
  // kept keys (for w) where LDS allows: the decode instantiation; the prefill
  // one writes the kept scores to w during the selection instead, to fit more
  // blocks
  __shared__ uint32_t s_keep[PCAP > 0 ? 4096 : 1];
  uint32_t* s_selkey = PCAP > 0 ? s_keep : nullptr;
  __shared__ int s_tmp[SelTmp<NT>::kSize];
  int32_t* s_selpos = reinterpret_cast<int32_t*>(s_hist);

  // prefill rows in descending order within each sequence: later rows see
  // more positions, and the longest selections then start first instead of
  // forming the launch's tail
  const int64_t bi = blockIdx.x;
  const int64_t nq = (int64_t)a.num_q * a.hq;  // selection rows per sequence
  const int64_t row = a.num_q > 1 ? (bi / nq) * nq + (nq - 1 - bi % nq) : bi;
  const int b = (int)(row / nq), i = (int)((row % nq) / a.hq);
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, a.num_q, b, i, cap);
  const int n = (int)rg.n;  // <= max_pages * block_size, which fits in int32
  // Global reads in flight per thread while LDS is filled: 4096 / NT (16 for
  // 256 threads), all issued before any is used. A decode row runs as one
  // block on its own, so its fills are latency-bound; prefill rows, three
  // blocks per CU, gain as well (fewer, longer waits on the score rows).
  constexpr int FU = kFillU<NT>;
  const float* srow = a.scores + row * a.ld;
  const int tid = threadIdx.x;
  // Without room for the kept keys in LDS, the final selection writes the kept
  // scores to w itself, from the keys it holds in registers.
  float* const w_out = (PCAP == 0 && a.w) ? a.w + row * a.topk : nullptr;
  // the final selection's outputs (DIRECT: the row's idx and w themselves)
  constexpr bool direct = DIRECT;
  int32_t* const f_pos = DIRECT ? a.idx + row * a.topk : s_selpos;
  uint32_t* const f_key = DIRECT ? nullptr : s_selkey;
  float* const f_w = DIRECT ? (a.w ? a.w + row * a.topk : nullptr) : w_out;

  if (FULL && a.n_sel_pages > 0) {
    // ---- block pruning: top pages by maximum score, then exact top-k inside
    const int n_pg = (n + kBlockSize - 1) / kBlockSize;
    const int P = (int)(n_pg < a.n_sel_pages ? n_pg : a.n_sel_pages);
    if (a.page_max) {
      const float* pm = a.page_max + row * a.max_pages;
      if (n_pg <= KCAP) {
        for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
        __syncthreads();
        for_keys<NT, FU>(GlobalPageMax{pm}, n_pg, [&](int g, uint32_t k) {
          s_keys[g] = k;
          atomicAdd(&s_hist[k >> (32 - kHistBits)], 1u);
        });
        __syncthreads();
        select_topk<NT>(LdsKeys{s_keys, nullptr, 0}, n_pg, P, s_hist, s_selpos, s_selkey, nullptr, s_tmp, true);
      } else {
        select_topk<NT>(GlobalPageMax{pm}, n_pg, P, s_hist, s_selpos, s_selkey, nullptr, s_tmp);
      }
    } else if (n_pg <= KCAP) {
      // page maxima from the score row: one thread per page, over valid positions
      for (int g = tid; g < n_pg; g += NT) s_keys[g] = PageMaxOfScores{srow, (int)rg.p}.key(g);
      __syncthreads();
      select_topk<NT>(LdsKeys{s_keys, nullptr, 0}, n_pg, P, s_hist, s_selpos, s_selkey, nullptr, s_tmp);
    } else {
      select_topk<NT>(PageMaxOfScores{srow, (int)rg.p}, n_pg, P, s_hist, s_selpos, s_selkey, nullptr, s_tmp);
    }
    for (int e = tid; e < P; e += NT) s_pages[e] = s_selpos[e];
    __syncthreads();
    // candidate positions of the kept pages, ascending; only the page holding
    // the query can be partial, and it is the last one in ascending order
    int m = P * kBlockSize;
    if (P > 0 && s_pages[P - 1] == (int)(rg.p >> 6)) m -= (kBlockSize - 1) - (rg.p & 63);
    const int K = (int)(m < a.topk ? m : a.topk);
    if (PCAP > 0 && m <= PCAP && m <= KCAP) {
      const KeptPageScores kept{srow, s_pages};
      for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
      __syncthreads();
      for_keys<NT, FU>(kept, m, [&](int e, uint32_t k) {
        s_keys[e] = k;
        s_pos[e] = kept.at(e);
        atomicAdd(&s_hist[k >> (32 - kHistBits)], 1u);
      });
      __syncthreads();
      select_topk<NT>(LdsKeys{s_keys, s_pos, 0}, m, K, s_hist, f_pos, f_key, f_w, s_tmp, true);
    } else {
      select_topk<NT>(KeptPageScores{srow, s_pages}, m, K, s_hist, f_pos, f_key, f_w, s_tmp);
    }
    write_row<NT>(a, row, K, s_selpos, s_selkey, srow, w_out != nullptr, direct);
    return;
  }

  // ---- exact top-k over every position 0..p
  const int K = (int)(n < a.topk ? n : a.topk);
  if (n <= a.topk) {
    keep_all<NT>(GlobalScores{srow}, n, f_pos, f_key, f_w);
  } else if (!FULL || n <= KCAP) {
    // the fill also builds the first radix pass's histogram
    for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
    __syncthreads();
    for_keys<NT, FU>(GlobalScores{srow}, n, [&](int e, uint32_t k) {
      s_keys[e] = k;
      atomicAdd(&s_hist[k >> (32 - kHistBits)], 1u);
    });
    __syncthreads();
    select_topk<NT, !FULL>(LdsKeys{s_keys, nullptr, 0}, n, K, s_hist, f_pos, f_key, f_w, s_tmp, true);
  } else if constexpr (FULL) {
    if constexpr (PCAP == 0) {
      // A prefill row longer than the LDS key buffer: the first-digit
      // histogram from the score row, then, in position order, every score
      // whose first digit reaches the threshold digit d into LDS as (key,
      // position) pairs; the select finishes over those (two passes over the
      // row instead of one per radix digit and one to compact). Falls through
      // to the pass-per-digit select when the pairs do not fit.
      for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
      __syncthreads();
      for_keys<NT, FU>(GlobalScores{srow}, n,
                   [&](int, uint32_t k) { atomicAdd(&s_hist[k >> (32 - kHistBits)], 1u); });
      __syncthreads();
      int above, in_bin;
      const int d = find_digit<NT, 4096>([&](int bin) { return s_hist[bin]; }, K, s_tmp, &above, &in_bin);
      constexpr int CC = KCAP / 2;  // (key, position) pairs that fit in s_keys
      if (above + in_bin <= CC) {   // block-uniform
        uint32_t* ck = s_keys;
        int32_t* cp = reinterpret_cast<int32_t*>(s_keys + CC);
        // keep keys of first digit >= d: key > (d << 20) - 1, or every key for d = 0
        const uint32_t lo = (uint32_t)d << (32 - kHistBits);
        ordered_compact<NT>(GlobalScores{srow}, n, d ? lo - 1u : 0u, d ? 0 : INT32_MAX, cp, ck, nullptr,
                        s_tmp);
        const int m = above + in_bin;
        uint32_t T;
        int r;
        radix_select<NT>(LdsKeys{ck, cp, 0}, m, 1, lo, ~0u << (32 - kHistBits), K - above, s_hist, s_tmp,
                     &T, &r);
        ordered_compact<NT>(LdsKeys{ck, cp, 0}, m, T, r, f_pos, f_key, f_w, s_tmp);
        write_row<NT>(a, row, K, s_selpos, s_selkey, srow, w_out != nullptr, direct);
        return;
      }
    }
    int m = -1;
    if (PCAP > 0 && a.cand_key && n >= a.long_row_min) {
      m = gather_candidates_spec<NT>(a, row, n, s_keys, s_pos, PCAP < KCAP ? PCAP : KCAP, s_tmp);
      if (MANY_SLICES && m == -2)
        m = gather_candidates_wave<NT>(a, row, n, s_keys, s_pos, PCAP < KCAP ? PCAP : KCAP,
                                       reinterpret_cast<int*>(s_hist), s_tmp);
      if (m == -2)
        m = gather_candidates<NT>(a, row, n, s_keys, s_pos, PCAP < KCAP ? PCAP : KCAP,
                              reinterpret_cast<int*>(s_hist), s_tmp);
    }
    if (m >= K) {
      // every candidate has a first digit >= the threshold digit t; the
      // `above` ones with a larger digit are all kept, and the radix select
      // continues at the second digit among those whose first digit is t
      const uint32_t t = (uint32_t)a.thresh[row];
      const int above = a.above[row];
      uint32_t T;
      int r;
      radix_select<NT>(LdsKeys{s_keys, s_pos, 0}, m, 1, t << (32 - kHistBits), ~0u << (32 - kHistBits), K - above, s_hist,
                   s_tmp, &T, &r);
      ordered_compact<NT>(LdsKeys{s_keys, s_pos, 0}, m, T, r, f_pos, f_key, f_w, s_tmp);
    } else {
      select_topk<NT>(GlobalScores{srow}, n, K, s_hist, f_pos, f_key, f_w, s_tmp);
    }
  }
  write_row<NT>(a, row, K, s_selpos, s_selkey, srow, w_out != nullptr, direct);
}

hipError_t launch_select(const SelectArgs& a, bool prefill_rows, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.num_q * a.hq;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;  // bound on every row's n
  const bool direct = a.page_mask == nullptr;
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(threads), 0, s, a);
  };
  if (prefill_rows) {
    constexpr int NT = kPrefillSelectThreads;
    const bool short_rows = a.n_sel_pages == 0 && cap <= kPrefillKeyCap;
    if (short_rows && direct) go(select_kernel<kPrefillKeyCap, 0, false, true, NT>, NT);
    else if (short_rows) go(select_kernel<kPrefillKeyCap, 0, false, false, NT>, NT);
    else if (direct) go(select_kernel<kPrefillKeyCap, 0, true, true, NT>, NT);
    else go(select_kernel<kPrefillKeyCap, 0, true, false, NT>, NT);
  } else {
    constexpr int NT = kDecodeSelectThreads;
    constexpr int KC = kDecodeKeyCap, PC = kDecodePosCap;
    const bool short_rows = a.n_sel_pages == 0 && cap <= kDecodeKeyCap;
    const bool many = a.cand_key && (cap + kCollectBlock - 1) / kCollectBlock > 32;
    if (short_rows && direct) go(select_kernel<KC, PC, false, true, NT>, NT);
    else if (short_rows) go(select_kernel<KC, PC, false, false, NT>, NT);
    else if (many && direct) go(select_kernel<KC, PC, true, true, NT, true>, NT);
    else if (many) go(select_kernel<KC, PC, true, false, NT, true>, NT);
    else if (direct) go(select_kernel<KC, PC, true, true, NT>, NT);
    else go(select_kernel<KC, PC, true, false, NT>, NT);
  }
  return hipGetLastError();
}

}  // namespace tis
