// score.hip -- indexer scoring kernels for gfx950.
//
// Scores are the plain dot product of a compressed query row with the
// compressed key of every causal position ("Day-0 Inference Adaptation of
// Ultra-Large-Scale MoE Models on Domestic AI Accelerators", section 4.1, step
// 1), read through the page table of the block-organised cache ("Day-0
// Inference Adaptation for Ultra-Large MoE Models on Domestic GPUs", section
// "Reorganizing KV Cache Layout").
//
// Decode (one query row per sequence) is a paged GEMV: every key byte is read
// once and used for one multiply-add, so the kernel is bound by HBM bandwidth.
// A wave reads a 64-row page as d_c/8 contiguous 1 KiB loads (one 16-byte
// segment per lane), forms per-lane partial dot products, and a DPP butterfly
// inside each group of d_c/8 lanes both reduces and scatters, leaving every
// lane with the full score of one row. Optional epilogues, fused so that the
// scores are not read back: per-page maxima for block pruning, and for long
// rows the first-digit histogram that the selection starts from (an LDS
// histogram per block whose nonzero bins are added into the row's histogram).
//
// Prefill (many query rows) is a GEMM with a causal mask: bf16 MFMA
// 16x16x32 tiles, keys as M, queries as N, d_c as K, the key tile staged in
// LDS; chunks strictly above the diagonal are skipped and positions after each
// row's query are not written.
#include <atomic>

#include "tis_common.h"
#include "tis_internal.h"

namespace tis {

constexpr int kScoreChunk = 512;  // keys per prefill scorer block (two tiles of 256)

// ------------------------------------------------------------ decode scorer

__device__ __forceinline__ float dot8(const float* q, u32x4 d) {
  float s = q[0] * bf16_lo(d.x);
  s = fmaf(q[1], bf16_hi(d.x), s);
  s = fmaf(q[2], bf16_lo(d.y), s);
  s = fmaf(q[3], bf16_hi(d.y), s);
  s = fmaf(q[4], bf16_lo(d.z), s);
  s = fmaf(q[5], bf16_hi(d.z), s);
  s = fmaf(q[6], bf16_lo(d.w), s);
  s = fmaf(q[7], bf16_hi(d.w), s);
  return s;
}

// One butterfly stage over V partial sums held by groups of 2*(V/2) lanes: the
// lane whose decision bit (value V/2 of its segment index) is set keeps the
// upper half, its partner the lower half, and each adds what the partner sends.
template <int V, int CTRL>
__device__ __forceinline__ void butterfly_stage(float* v, int seg) {
  const bool up = (seg & (V / 2)) != 0;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    const float send = up ? v[i] : v[i + V / 2];
    const float keep = up ? v[i + V / 2] : v[i];
    v[i] = keep + dpp<CTRL>(send);
  }
}

// After the reduction lane `seg` of each group holds the complete sum of value
// index `seg`.
template <int LPR>
__device__ __forceinline__ float butterfly_reduce(float* v, int seg) {
  if constexpr (LPR == 16) {
    butterfly_stage<16, kDppRowMirror>(v, seg);
    butterfly_stage<8, kDppRowHalfMirror>(v, seg);
    butterfly_stage<4, kDppXor3>(v, seg);
    butterfly_stage<2, kDppXor1>(v, seg);
  } else {
    butterfly_stage<8, kDppRowHalfMirror>(v, seg);
    butterfly_stage<4, kDppXor3>(v, seg);
    butterfly_stage<2, kDppXor1>(v, seg);
  }
  return v[0];
}

#ifndef TIS_SCORE_NT
#define TIS_SCORE_NT 1  // streaming (non-temporal) loads of the compressed keys
#endif

template <int LPR>
__device__ __forceinline__ void load_page(u32x4* d, const uint16_t* base, int lane) {
#pragma unroll
  for (int k = 0; k < LPR; ++k) {
    const u32x4* p = reinterpret_cast<const u32x4*>(base + k * 512 + lane * 8);
#if TIS_SCORE_NT
    d[k] = __builtin_nontemporal_load(p);
#else
    d[k] = *p;
#endif
  }
}

// Each wave streams a run of PPW pages. Page ids are read up front, and the
// loads of page t+1 are issued (behind a scheduling barrier) before page t is
// reduced, so every wave keeps two pages of loads in flight. With HIST, rows of
// at least long_row_min positions also count the first 12-bit digit of every
// score in an LDS histogram (cleared while the first page loads are in
// flight); the block then adds its nonzero bins into the row histogram, which
// a clear kernel zeroed before this launch.
template <int DC, bool PMAX, bool HIST, int PPB>
__global__ __launch_bounds__(256) void score_decode_kernel(ScoreDecodeArgs a) {
  constexpr int LPR = DC / 8;    // lanes per key row (16 B each)
  constexpr int RPL = 64 / LPR;  // rows per wave-wide 1 KiB load
  static_assert(PPB % 4 == 0, "pages per block split evenly over 4 waves");
  constexpr int PPW = PPB / 4;

  const int b = blockIdx.y;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  const int64_t n_pg = (rg.n + kBlockSize - 1) / kBlockSize;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gb = (int64_t)blockIdx.x * PPB;
  if (gb >= n_pg) return;  // the whole block lies past the row: uniform exit
  const bool hist = HIST && rg.n >= a.long_row_min;  // block-uniform
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[HIST ? kHistBins : 4];

  const int64_t g0 = gb + wave * PPW;
  const bool active = g0 < n_pg;  // wave-uniform
  const int npw = active ? (int)(n_pg - g0 < PPW ? n_pg - g0 : PPW) : 0;
  const int seg = lane % LPR, rsub = lane / LPR;

  // the query slice first: the wait counter drains in issue order
  float qf[8];
  {
    const u32x4 qv = *reinterpret_cast<const u32x4*>(a.q_comp + (int64_t)b * DC + seg * 8);
    qf[0] = bf16_lo(qv.x); qf[1] = bf16_hi(qv.x);
    qf[2] = bf16_lo(qv.y); qf[3] = bf16_hi(qv.y);
    qf[4] = bf16_lo(qv.z); qf[5] = bf16_hi(qv.z);
    qf[6] = bf16_lo(qv.w); qf[7] = bf16_hi(qv.w);
  }
  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  const uint16_t* pbase[PPW];
#pragma unroll
  for (int t = 0; t < PPW; ++t) {
    int pid = t < npw ? pt[g0 + t] : 0;
    pid = pid < 0 ? 0 : (pid >= a.num_phys ? a.num_phys - 1 : pid);
    pbase[t] = a.k_comp + (int64_t)pid * kBlockSize * DC;
  }
  __builtin_amdgcn_sched_barrier(0);
  float* srow = a.scores + (int64_t)b * a.ld;

  // a wave past the row (only in a row's last block) reads page 0 of the pool
  // and uses nothing of it: the loads stay unconditional, so that the wait
  // counts stay exact
  u32x4 buf[2][LPR];
  load_page<LPR>(buf[0], pbase[0], lane);
  if (HIST && hist) {
#pragma unroll
    for (int k = 0; k < kHistBins / 1024; ++k)
      *reinterpret_cast<u32x4*>(&s_hist[(k * 256 + tid) * 4]) = u32x4{0u, 0u, 0u, 0u};
    lds_barrier();  // the page loads stay in flight
  }
#pragma unroll
  for (int t = 0; t < PPW; ++t) {
    if (t >= npw) break;  // wave-uniform
    if (t + 1 < npw) load_page<LPR>(buf[(t + 1) & 1], pbase[t + 1], lane);
    __builtin_amdgcn_sched_barrier(0);
    float part[LPR];
#pragma unroll
    for (int k = 0; k < LPR; ++k) part[k] = dot8(qf, buf[t & 1][k]);
    const float s = butterfly_reduce<LPR>(part, seg);
    const int64_t g = g0 + t;
    const int64_t j = g * kBlockSize + seg * RPL + rsub;
    const bool valid = j <= rg.p;
    if (valid) srow[j] = s;
    if constexpr (HIST) {
      if (hist && valid) atomicAdd(&s_hist[score_key(s) >> (32 - kHistBits)], 1u);
    }
    if constexpr (PMAX) {
      const float m = wave_max(valid ? s : -INFINITY);
      if (lane == 0) a.page_max[(int64_t)b * a.max_pages + g] = m;
    }
  }
  if (HIST && hist) {
    lds_barrier();  // every wave's bin updates are done
    add_row_hist(s_hist, a.row_hist + (int64_t)b * kRowHistWords);
  }
}

// The scan with page maxima (block pruning) for large tables, with the score
// stores taken out of the key stream: a block holds the scores of its pages in
// LDS and writes them, as 16-byte stores, when all its pages are done, and the
// launcher sizes the blocks so that one round of them (three per compute unit)
// covers the table. (Score stores mixed into the key loads cost the scan about
// 15% of its read rate, and written at the block's end about a third of that;
// with blocks of unequal rows, as in ragged batches, the one round loses more
// to imbalance than that, so the histogramming scan keeps small blocks.) Wave
// w takes the block's pages w, w + 4, ...; lane i holds the physical id of the
// wave's i-th page, and the next page's loads are in flight while a page is
// reduced.
template <int DC>
__global__ __launch_bounds__(256, 3) void score_decode_pmax_kernel(ScoreDecodeArgs a) {
  constexpr int LPR = DC / 8;    // lanes per key row (16 B each)
  constexpr int RPL = 64 / LPR;  // rows per wave-wide 1 KiB load
  __shared__ __attribute__((aligned(16))) float s_sc[kMaxDeferPages * kBlockSize];

  const int b = blockIdx.y;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  const int64_t n_pg = (rg.n + kBlockSize - 1) / kBlockSize;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gb = (int64_t)blockIdx.x * a.ppb;
  if (gb >= n_pg) return;  // the whole block lies past the row: uniform exit
  const int nb = (int)(n_pg - gb < a.ppb ? n_pg - gb : a.ppb);  // <= kMaxDeferPages
  const int npw = nb > wave ? (nb - wave + 3) / 4 : 0;  // pages of this wave (<= 32)
  const int seg = lane % LPR, rsub = lane / LPR;

  float qf[8];
  {
    const u32x4 qv = *reinterpret_cast<const u32x4*>(a.q_comp + (int64_t)b * DC + seg * 8);
    qf[0] = bf16_lo(qv.x); qf[1] = bf16_hi(qv.x);
    qf[2] = bf16_lo(qv.y); qf[3] = bf16_hi(qv.y);
    qf[4] = bf16_lo(qv.z); qf[5] = bf16_hi(qv.z);
    qf[6] = bf16_lo(qv.w); qf[7] = bf16_hi(qv.w);
  }
  int pid = 0;
  if (lane < npw) {
    pid = a.page_table[(int64_t)b * a.max_pages + gb + wave + 4 * lane];
    pid = pid < 0 ? 0 : (pid >= a.num_phys ? a.num_phys - 1 : pid);
  }
  auto load = [&](u32x4 (&d)[LPR], int i) {  // i wave-uniform, < npw
    const uint16_t* base = a.k_comp + (int64_t)__builtin_amdgcn_readlane(pid, i) * kBlockSize * DC;
    load_page<LPR>(d, base, lane);
  };
  auto reduce = [&](const u32x4 (&d)[LPR], int i) {
    float part[LPR];
#pragma unroll
    for (int k = 0; k < LPR; ++k) part[k] = dot8(qf, d[k]);
    const float s = butterfly_reduce<LPR>(part, seg);
    const int t = wave + 4 * i;  // page of the block
    const int jl = seg * RPL + rsub;
    const int64_t g = gb + t;
    s_sc[t * kBlockSize + jl] = s;
    const float m = wave_max(g * kBlockSize + jl <= rg.p ? s : -INFINITY);
    if (lane == 0) a.page_max[(int64_t)b * a.max_pages + g] = m;
  };

  u32x4 b0[LPR], b1[LPR];
  if (npw > 0) load(b0, 0);
  for (int i = 0; i < npw; i += 2) {
    if (i + 1 < npw) load(b1, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    reduce(b0, i);
    if (i + 1 >= npw) break;
    if (i + 2 < npw) load(b0, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    reduce(b1, i + 1);
  }
  __syncthreads();  // every wave's scores are in LDS
  // the block's positions gb*64 .. up to the row's last: 16-byte stores, then
  // the partial last group of four one by one
  const int nv = (int)((rg.p + 1 - gb * kBlockSize) < (int64_t)nb * kBlockSize
                           ? (rg.p + 1 - gb * kBlockSize) : (int64_t)nb * kBlockSize);
  float* dst = a.scores + (int64_t)b * a.ld + gb * kBlockSize;
  for (int i = tid; i < nv / 4; i += 256)
    reinterpret_cast<f32x4*>(dst)[i] = reinterpret_cast<const f32x4*>(s_sc)[i];
  if (tid < (nv & 3)) dst[(nv & ~3) + tid] = s_sc[(nv & ~3) + tid];
}

// Decode scorer for several indexer heads (HQ <= 16) of one sequence: per page
// S^T = K (64 keys x d_c) . Qc^T (d_c x 16 heads) on bf16 MFMA 16x16x32, keys
// as M and heads as N, so that each compressed key is read once for all heads
// (a thin GEMM; still bound by the key bytes). A wave reads its pages as whole
// 1 KiB rows-contiguous loads (loads laid out as MFMA fragments, 16 rows x 64
// bytes each, stream about 15% slower), stores each page into its own LDS
// buffer with the 16-byte segments of row r XOR-swizzled by r mod 16, and
// reads the MFMA A fragments back (key 16m + c, dims 32k + 8(lane/16)): both
// directions touch 16 distinct segments per 16 lanes, so neither conflicts.
// The next page's loads are in flight while a page is computed. Results: lane
// (c, g) holds head c's scores of keys 16m + 4g .. +3.
template <int DC, bool PMAX, int PPB>
__global__ __launch_bounds__(256) void score_decode_mh_kernel(ScoreDecodeArgs a) {
  constexpr int KS = DC / 32;    // MFMA k-steps
  constexpr int SEG = DC / 8;    // 16-byte segments per key row
  constexpr int LPR = DC / 8;    // lanes per row in a 1 KiB load
  constexpr int RPL = 64 / LPR;  // rows per 1 KiB load
  constexpr int NL = 64 / RPL;   // 1 KiB loads per page
  static_assert(PPB % 4 == 0, "pages per block split evenly over 4 waves");
  constexpr int PPW = PPB / 4;
  __shared__ __attribute__((aligned(16))) u32x4 s_page[4][64 * SEG];  // one page per wave
  const int b = blockIdx.y;
  const int hq = a.hq;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const RowGeom rg = row_geom(a.seq_lens, a.q_start, 1, b, 0, cap);
  const int64_t n_pg = (rg.n + kBlockSize - 1) / kBlockSize;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g4 = lane >> 4;
  const int64_t g0 = (int64_t)blockIdx.x * PPB + wave * PPW;
  if (g0 >= n_pg) return;  // wave-uniform; the kernel has no block barrier
  const int npw = (int)(n_pg - g0 < PPW ? n_pg - g0 : PPW);
  u32x4* const lds = s_page[wave];

  // head c's compressed query (MFMA B operand: dims 32k + 8 g4 .. +7)
  bf16x8 qf[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < hq)
      v = *reinterpret_cast<const u32x4*>(a.q_comp + ((int64_t)b * hq + c) * DC + k * 32 + g4 * 8);
    qf[k] = __builtin_bit_cast(bf16x8, v);
  }
  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  const uint16_t* pbase[PPW];
#pragma unroll
  for (int t = 0; t < PPW; ++t) {
    int pid = t < npw ? pt[g0 + t] : 0;
    pid = pid < 0 ? 0 : (pid >= a.num_phys ? a.num_phys - 1 : pid);
    pbase[t] = a.k_comp + (int64_t)pid * kBlockSize * DC;
  }
  __builtin_amdgcn_sched_barrier(0);
  // load u: rows RPL*u + lane / LPR, segment lane % LPR
  const int lrow = lane / LPR, lseg = lane % LPR;
  auto load = [&](u32x4 (&d)[NL], const uint16_t* base) {
#pragma unroll
    for (int u = 0; u < NL; ++u)
      d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + u * 512 + lane * 8));
  };
  const bool store_head = c < hq;
  float* srow = a.scores + ((int64_t)b * hq + (store_head ? c : 0)) * a.ld;
  u32x4 buf[2][NL];
  load(buf[0], pbase[0]);
#pragma unroll
  for (int t = 0; t < PPW; ++t) {
    if (t >= npw) break;  // wave-uniform
    if (t + 1 < npw) load(buf[(t + 1) & 1], pbase[t + 1]);
    __builtin_amdgcn_sched_barrier(0);
    // the page into the wave's LDS buffer (the previous page's reads are done:
    // the wave's LDS operations complete in order, and the fences keep the
    // compiler from moving them across each other)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int r = RPL * u + lrow;
      lds[r * SEG + (lseg ^ (r & (SEG - 1)))] = buf[t & 1][u];
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    f32x4 acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * m + c;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const u32x4 v = lds[r * SEG + ((4 * k + g4) ^ (r & (SEG - 1)))];
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), qf[k],
                                                         acc[m], 0, 0, 0);
      }
    }
    const int64_t g = g0 + t;
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t j = g * kBlockSize + m * 16 + 4 * g4;
      if (store_head) {
        if (j + 3 <= rg.p) {
          *reinterpret_cast<f32x4*>(srow + j) = acc[m];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (j + i <= rg.p) srow[j + i] = acc[m][i];
        }
      }
      if constexpr (PMAX) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, j + i <= rg.p ? acc[m][i] : -INFINITY);
      }
    }
    if constexpr (PMAX) {
      mx = max_over_rows(mx);  // over the page's 64 keys of head c
      if (store_head && g4 == 0) a.page_max[((int64_t)b * hq + c) * a.max_pages + g] = mx;
    }
  }
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_score_decode(const ScoreDecodeArgs& a, hipStream_t s) {
  const bool pmax = a.page_max != nullptr, hist = a.row_hist != nullptr;
  if (pmax && hist) return hipErrorInvalidValue;  // pruned rows select from page maxima
  if (a.hq > 1) {  // several indexer heads: the MFMA scorer (no histogram epilogue)
    if (hist || a.hq > 16) return hipErrorInvalidValue;
    if ((reinterpret_cast<uintptr_t>(a.scores) & 15) || (a.ld & 3)) return hipErrorInvalidValue;
    constexpr int P = kPagesPerScoreBlock;
    const dim3 grid((unsigned)(((int64_t)a.max_pages + P - 1) / P), (unsigned)a.batch);
    if (a.d_c == 64) {
      if (pmax) hipLaunchKernelGGL((score_decode_mh_kernel<64, true, P>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((score_decode_mh_kernel<64, false, P>), grid, dim3(256), 0, s, a);
    } else {
      if (pmax) hipLaunchKernelGGL((score_decode_mh_kernel<128, true, P>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((score_decode_mh_kernel<128, false, P>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  // Page maxima over a large table: blocks that hold their scores until they
  // end, sized so that one round of them (three per compute unit) covers the
  // table (judged from its width, since the row lengths are on the device).
  if (pmax) {
    const int64_t per_round = 3 * (int64_t)device_cus();
    int64_t ppb = ((int64_t)a.batch * a.max_pages + per_round - 1) / per_round;
    ppb = (ppb + 3) / 4 * 4;
    if (ppb > kMaxDeferPages) ppb = kMaxDeferPages;
    if (ppb >= kMinDeferPages && !(reinterpret_cast<uintptr_t>(a.scores) & 15) && !(a.ld & 3)) {
      ScoreDecodeArgs d = a;
      d.ppb = (int)ppb;
      const dim3 grid((unsigned)(((int64_t)a.max_pages + ppb - 1) / ppb), (unsigned)a.batch), block(256);
      if (a.d_c == 64) hipLaunchKernelGGL((score_decode_pmax_kernel<64>), grid, block, 0, s, d);
      else hipLaunchKernelGGL((score_decode_pmax_kernel<128>), grid, block, 0, s, d);
      return hipGetLastError();
    }
  }
  // Histogramming blocks: wide ones when a single round of them (three per
  // compute unit, as the d_c = 128 kernel's registers allow) covers the table,
  // judged from its width since the row lengths are on the device.
  bool wide = true;
  if (hist) {
    const int64_t wide_blocks = (int64_t)a.batch *
        (((int64_t)a.max_pages + kPagesPerHistScoreBlockWide - 1) / kPagesPerHistScoreBlockWide);
    wide = wide_blocks <= 3 * (int64_t)device_cus();
  }
  // Without histograms: one page per wave when 16-page blocks would not give
  // every compute unit a block.
  const bool small = !hist && (int64_t)a.batch * (((int64_t)a.max_pages + kPagesPerScoreBlock - 1) /
                                                  kPagesPerScoreBlock) < (int64_t)device_cus();
  const int ppb = !hist ? (small ? kPagesPerScoreBlockSmall : kPagesPerScoreBlock)
                        : (wide ? kPagesPerHistScoreBlockWide : kPagesPerHistScoreBlockNarrow);
  const int64_t chunks = ((int64_t)a.max_pages + ppb - 1) / ppb;
  const dim3 grid((unsigned)chunks, (unsigned)a.batch), block(256);
  constexpr int P = kPagesPerScoreBlock, PS = kPagesPerScoreBlockSmall,
                HW = kPagesPerHistScoreBlockWide, HN = kPagesPerHistScoreBlockNarrow;
  if (a.d_c == 64) {
    if (pmax && small) hipLaunchKernelGGL((score_decode_kernel<64, true, false, PS>), grid, block, 0, s, a);
    else if (pmax) hipLaunchKernelGGL((score_decode_kernel<64, true, false, P>), grid, block, 0, s, a);
    else if (hist && wide) hipLaunchKernelGGL((score_decode_kernel<64, false, true, HW>), grid, block, 0, s, a);
    else if (hist) hipLaunchKernelGGL((score_decode_kernel<64, false, true, HN>), grid, block, 0, s, a);
    else if (small) hipLaunchKernelGGL((score_decode_kernel<64, false, false, PS>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((score_decode_kernel<64, false, false, P>), grid, block, 0, s, a);
  } else {
    if (pmax && small) hipLaunchKernelGGL((score_decode_kernel<128, true, false, PS>), grid, block, 0, s, a);
    else if (pmax) hipLaunchKernelGGL((score_decode_kernel<128, true, false, P>), grid, block, 0, s, a);
    else if (hist && wide) hipLaunchKernelGGL((score_decode_kernel<128, false, true, HW>), grid, block, 0, s, a);
    else if (hist) hipLaunchKernelGGL((score_decode_kernel<128, false, true, HN>), grid, block, 0, s, a);
    else if (small) hipLaunchKernelGGL((score_decode_kernel<128, false, false, PS>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((score_decode_kernel<128, false, false, P>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------- prefill scorer

// Block: 64 query rows (16 per wave) x one chunk of kScoreChunk keys, walked in
// tiles of two pages. Each tile's compressed keys are staged in LDS once for
// the four waves; the chunk's page ids are read up front, and the next tile's
// 16-byte loads are in flight while the current tile is scored. The output is
// the dominant traffic (4 bytes per causal pair): with keys as the MFMA rows a
// lane holds 4 consecutive scores of one query row, so a wave's 16 rows x 64
// keys of a page pass through a small LDS buffer, after which each store
// instruction writes 4 whole 256-byte row segments (a direct 16-byte store per
// lane would write 16 rows x 64 bytes per instruction, 15% slower overall).
template <int DC>
__global__ __launch_bounds__(256) void score_prefill_kernel(ScorePrefillArgs a) {
  constexpr int TP = 2;                     // pages per key tile
  constexpr int KS = DC / 32;               // MFMA k-steps
  constexpr int KP = DC + 8;                // LDS row pitch in bf16 (16-byte pad)
  constexpr int SEG_ROW = DC / 8;           // 16-byte segments per key row
  constexpr int SPT = TP * 64 * SEG_ROW / 256;  // segments per thread
  constexpr int UPP = SPT / TP;             // ... of which per page
  constexpr int TK = 64 * TP;               // keys per tile
  constexpr int TPC = kScoreChunk / TK;     // tiles per chunk
  constexpr int OP = 68;                    // staged output row pitch in floats
  __shared__ __attribute__((aligned(16))) uint16_t kt[TP * 64 * KP];
  __shared__ __attribute__((aligned(16))) float ost[4 * 16 * OP];
  const int b = blockIdx.z;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g4 = lane >> 4;
  // rows of a sequence: (query row, indexer head) pairs, row r at the
  // position of query row r / hq
  const int nr = a.num_q * a.hq;
  auto geom = [&](int r) { return row_geom(a.seq_lens, a.q_start, a.num_q, b, r / a.hq, cap); };

  // Row blocks along x: consecutive blocks go to the 8 XCDs in turn, so each
  // XCD takes every eighth row block and the causal triangle's work spreads
  // evenly over them. Chunks along y, counted down from the row block's
  // diagonal: every block of a low y has work and is dispatched first, and
  // the blocks beyond a row block's chunks (which only read its geometry and
  // exit) come last, instead of holding slots that blocks with work wait for.
  const int row0 = blockIdx.x * 64;
  // positions grow with the row index: the block's last valid row sees furthest
  const int last_row = min(row0 + 63, nr - 1);
  const RowGeom last = geom(last_row);
  if (last.p < 0) return;  // no row of the block sees a position
  if (last.n <= a.skip_n) return;  // rows whose scores nobody reads
  if ((int64_t)blockIdx.y > last.p / kScoreChunk) return;  // beyond the row block's chunks
  const int64_t chunk0 = (last.p / kScoreChunk - (int64_t)blockIdx.y) * kScoreChunk;
  int64_t nkt64 = (last.p - chunk0) / TK + 1;
  nkt64 = nkt64 < TPC ? nkt64 : TPC;
  const int nkt = (int)nkt64;  // key tiles of the chunk that some row of the block sees

  // this wave's query rows (MFMA B operand), issued before the first page loads
  const int wrow0 = row0 + wave * 16;
  bf16x8 af[KS];
  {
    const int r = min(wrow0 + c, nr - 1);
    const uint16_t* qrow = a.q_comp + ((int64_t)b * nr + r) * DC;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      af[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + k * 32 + g4 * 8));
  }
  // physical ids of the chunk's pages, all loaded up front (clamped into the pool)
  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  int pid[TP * TPC];
#pragma unroll
  for (int p = 0; p < TP * TPC; ++p) {
    const int64_t g = (chunk0 >> 6) + p;
    const int v = g < a.max_pages ? pt[g] : 0;
    pid[p] = v < 0 ? 0 : (v >= a.num_phys ? a.num_phys - 1 : v);
  }
  // the 16-byte segments of key tile t, held in registers until stored to LDS
  auto fetch = [&](int t, u32x4 (&seg)[SPT]) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int p = u / UPP;                            // page of this segment
      const int in_page = tid + 256 * (u % UPP);        // segment index within the page
      const int row = in_page / SEG_ROW, part = in_page % SEG_ROW;
      int id = pid[p];
#pragma unroll
      for (int q = 1; q < TPC; ++q) id = t == q ? pid[TP * q + p] : id;
      seg[u] = *reinterpret_cast<const u32x4*>(a.k_comp + ((int64_t)id * kBlockSize + row) * DC +
                                               part * 8);
    }
  };
  auto stage = [&](const u32x4 (&seg)[SPT]) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int p = u / UPP;
      const int in_page = tid + 256 * (u % UPP);
      const int row = in_page / SEG_ROW, part = in_page % SEG_ROW;
      *reinterpret_cast<u32x4*>(&kt[(p * 64 + row) * KP + part * 8]) = seg[u];
    }
  };

  // 16-byte stores need 16-byte aligned rows
  const bool vec = (a.ld % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
  const int wlast = min(wrow0 + 15, nr - 1);
  const int64_t wl_p = wrow0 < nr ? geom(wlast).p : -1;
  // the rows this lane stores: 4k + lane/16 of the wave's 16
  int64_t p_st[4];
  float* srow[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = wrow0 + 4 * k + (lane >> 4);
    p_st[k] = r < nr ? geom(r).p : -1;
    srow[k] = a.scores + ((int64_t)b * nr + (r < nr ? r : 0)) * a.ld;
  }
  float* const ow = ost + wave * 16 * OP;

  u32x4 seg[SPT];
  fetch(0, seg);
  for (int t = 0; t < nkt; ++t) {
    stage(seg);
    __syncthreads();
    if (t + 1 < nkt) fetch(t + 1, seg);  // in flight while this tile is computed
    const int64_t k0 = chunk0 + TK * t;
#pragma unroll
    for (int p = 0; p < TP; ++p) {
      const int64_t g = (k0 >> 6) + p;
      if (g * kBlockSize > wl_p) break;  // the rest of the tile is masked for this wave
      f32x4 acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint16_t* krow = &kt[(p * 64 + nt * 16 + c) * KP];
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const bf16x8 bf =
              __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + k * 32 + g4 * 8));
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[k], acc[nt], 0, 0, 0);
        }
      }
      // rows c, keys 16nt + 4g4 + i in; rows 4k + lane/16, keys 4(lane%16) + i out.
      // The buffer is the wave's own: wave-scope fences keep the compiler from
      // moving these accesses across each other (the wave's LDS operations
      // then complete in program order)
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        *reinterpret_cast<f32x4*>(&ow[c * OP + nt * 16 + g4 * 4]) = acc[nt];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&ow[(4 * k + (lane >> 4)) * OP + 4 * c]);
        const int64_t j = g * kBlockSize + 4 * c;
        if (vec && j + 3 <= p_st[k]) {
          *reinterpret_cast<f32x4*>(srow[k] + j) = v;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (j + i <= p_st[k]) srow[k][j + i] = v[i];
        }
      }
    }
    __syncthreads();  // the tile's LDS reads are done before the next is stored
  }
}

hipError_t launch_score_prefill(const ScorePrefillArgs& a, hipStream_t s) {
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int64_t nr = (int64_t)a.num_q * a.hq;
  if ((cap + kScoreChunk - 1) / kScoreChunk > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)((nr + 63) / 64), (unsigned)((cap + kScoreChunk - 1) / kScoreChunk),
            (unsigned)a.batch);
  if (a.d_c == 64)
    hipLaunchKernelGGL((score_prefill_kernel<64>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((score_prefill_kernel<128>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tis
