// prefill.hip -- prefill attention over the shared sparse mask, for gfx950.
//
// In prefill every position of the context is a query row, so neighbouring
// rows select largely the same pages. The decode path gathers each row's
// selected K/V rows on its own; here a workgroup takes a run of consecutive
// query rows, turns their index lists into the per-(row, page) bitmask ("Day-0
// Inference Adaptation for Ultra-Large MoE Models on Domestic GPUs", sections
// "Operatorizing Index Selection" and "Separate Paths for Prefill and Decode":
// one sparse-mask representation shared by both paths, and batched fused
// operators with large blocked matrix products for the compute-bound prefill;
// "Day-0 Adaptation for Trillion-Parameter MoE Models", section IV: the
// compute-heavy prefill kernel over the gathered pages), and streams every
// page that any of its rows selected through LDS once, for all of them:
//   S^T = K Q^T        bf16 MFMA 16x16x32, 64 keys x 16 (row, head) columns;
//   masked online softmax per (row, head) in fp32, keys outside the row's
//   selection get weight zero;
//   O^T += V^T P^T     bf16 MFMA, P rounded to bf16 (its rounded values form
//   the normaliser, as in the decode path).
// The result equals exact softmax attention over each row's selected set: a
// selected key is one whose bit is set, and masked keys contribute exactly 0.
//
// Work split: an M-tile is one query row with 16 of its heads (head tile ht).
// A workgroup of 4 waves holds 8 M-tiles (2 per wave): 8 / HT rows of HT head
// tiles, so that every page staged in LDS serves 8 M-tiles. Two workgroups
// share a CU (LDS of about 79 KB each, at most 256 VGPRs per wave), so that
// each SIMD runs one wave of each: while one workgroup waits at its per-page
// barrier or on LDS, the other's wave issues.
// LDS: the K and V pages (layouts below), each in two buffers so that page g+1
// is loaded while page g is computed, the page's bias rows (each wave's own),
// and the bitmask of the workgroup's rows. Both pages go from global memory
// straight into LDS; V^T fragments come from transposing LDS reads.
#include <type_traits>

#include "tis_common.h"
#include "tis_internal.h"

namespace tis {

constexpr int kTPW = 2;         // M-tiles per wave
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;
constexpr float kSlack = 8.0f;  // log2 headroom of the softmax weights

// LDS layouts of a page:
//   K   rows of 256 bytes (key r, 128 dims: 16 slots of 16 bytes) whose slots
//       are XOR-swizzled by the row, slot s of key r at slot s ^ (r % 16), so
//       that the 16 lanes of a fragment read, each in a different row, touch 16
//       different slots;
//   V   key-major rows as in the cache, at a pitch of 18 slots (288 bytes: 8
//       banks further per row), so that the four rows x four 8-byte pieces a
//       16-lane group of a transposing read gathers cover the 32 banks once,
//       and so that every read's address is a per-lane base plus a constant
//       for the chunk, the dim tile and the half. (At 17 slots, 4 banks per
//       row, the pieces of neighbouring rows collided.)
constexpr int kVRowSlots = 18;
constexpr int kVPitch = kVRowSlots * 8;            // bf16 elements per V row in LDS
constexpr int kVSlots = kVRowSlots * kBlockSize;   // 16-byte slots per V page in LDS (2 per row unused)
__device__ __forceinline__ int k_lds_index(int r, int seg) { return r * 128 + 8 * (seg ^ (r & 15)); }

template <int ROWS, int WAVES>
struct PrefillLds {
  uint16_t k[2][kBlockSize * kHeadDim];
  uint16_t v[2][kVSlots * 8];                 // [buffer][key at pitch kVPitch]
  uint64_t mask[ROWS * kPrefillMaskPages];    // [row in group][page]
  float bias[WAVES][kTPW][kBlockSize];        // [wave][M-tile][key]: 0 or -inf
  int32_t ppid[kPrefillMaskPages];            // physical page of the group's n-th page
  int16_t plist[kPrefillMaskPages];           // logical page of the group's n-th page
  int32_t wcount[kPrefillMaskPages / 64];     // selected pages per 64-page span
  int32_t max_page;                           // highest page the group's lists name
};

// Pages go from global memory straight into LDS (16 bytes per lane; a wave
// writes 64 consecutive 16-byte slots): lane t of the block fetches whatever
// its slot holds in the layouts above.
// A thread's byte offsets within a page (K: its four rows' swizzled slots; V:
// its slots of the padded key-major layout), computed once: unsigned 32-bit
// values beside the page's uniform base, so that the loads take the
// scalar-base address form.
template <int PW>
struct PageOffsets {
  static constexpr int NT = 64 * PW, KQ = 1024 / NT, NC = kVSlots / 64, VQ = (NC + PW - 1) / PW;
  uint32_t k[KQ], v[VQ];
  int wave;  // wave-uniform
  __device__ explicit PageOffsets(int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const int r = NT / 16 * q + tid / 16;
      k[q] = 2u * (uint32_t)(r * kHeadDim + 8 * ((tid & 15) ^ (r & 15)));
    }
#pragma unroll
    for (int q = 0; q < VQ; ++q) {
      const int u = 64 * (q * PW + wave) + lane, r = u / kVRowSlots;
      const int slot = u - kVRowSlots * r;
      v[q] = 2u * (uint32_t)(r * kHeadDim + 8 * (slot >= 16 ? slot - 16 : slot));  // padding: a copy
    }
  }
};
// One direct load: lane l's 16 bytes at base + voff (base wave-uniform, voff
// an unsigned byte offset: the scalar-base form) land at LDS byte address
// lds + 16 l. It is issued from an asm statement: the compiler, which cannot
// tell the two page buffers apart, would otherwise make every transposing V
// read wait for the next page's loads still in flight (3-6 us of the
// attention at 8K tokens). The instruction has no register results; the page
// loop waits for its loads itself (s_waitcnt) before the barrier that
// publishes the page, and M0 takes the LDS address one instruction ahead, as
// the hardware asks.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int PW>
__device__ __forceinline__ void load_page_k(const uint16_t* kpage, uint16_t* k,
                                            const PageOffsets<PW>& o) {
#pragma unroll
  for (int q = 0; q < PageOffsets<PW>::KQ; ++q)  // the wave's four rows
    dma16(kpage, o.k[q], lds_addr(k + (64 * PW / 16 * q + o.wave * 4) * kHeadDim));
}
// V: the wave's chunk ch holds slots 64 ch .. 64 ch + 63, slot u being slot
// u % 18 of key u / 18 (slots 16 and 17 of a row are padding and take copies
// of its slots 0 and 1)
template <int PW>
__device__ __forceinline__ void load_page_v(const uint16_t* vpage, uint16_t* v,
                                            const PageOffsets<PW>& o) {
  using O = PageOffsets<PW>;
#pragma unroll
  for (int q = 0; q < O::VQ; ++q) {
    const int ch = q * PW + o.wave;
    if (ch < O::NC)  // wave-uniform
      dma16(vpage, o.v[q], lds_addr(v + 64 * 8 * ch));
  }
}

template <int HT, int PW, bool LSE, bool WIN>
__global__ __launch_bounds__(64 * PW, 2) void prefill_attend_kernel(AttendArgs a) {
  constexpr int kPT = 64 * PW;
  static_assert(kPT >= kPrefillMaskPages, "one thread per page in the page scan");
  constexpr int kRows = PW * kTPW;    // M-tiles per workgroup: the rows at HT = 1
  constexpr int QB = kRows / HT;      // query rows per workgroup
  __shared__ __attribute__((aligned(16))) PrefillLds<kRows, PW> L;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int groups = (a.num_q + QB - 1) / QB;
  // Heavy groups (late rows: long contexts) first. Neighbouring groups select
  // nearly the same pages, and consecutive workgroups go to the 8 XCDs in
  // turn, each with its own L2: so runs of 8 consecutive groups go to one XCD
  // (in each 64 workgroups, u % 8 picks the run, in reverse order every other
  // 64 so that no XCD always takes the heaviest run, and (u / 8) % 8 the
  // member); past the last whole 64 groups the order is plain. With several
  // indexer heads a workgroup takes one head's selections and query heads.
  const int u = (int)(blockIdx.x % groups), g64 = groups - groups % 64;
  const int run = ((u / 64) & 1) ? 7 - u % 8 : u % 8;
  const int gi = groups - 1 - (u < g64 ? 64 * (u / 64) + 8 * run + (u / 8) % 8 : u);
  const int gh = (int)((blockIdx.x / groups) % a.idx_heads);
  const int b = (int)(blockIdx.x / ((int64_t)groups * a.idx_heads));
  const int q0 = gi * QB;
  const int nrows = min(QB, a.num_q - q0);
  const int H = a.num_heads;  // query heads per selection row
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  // selection row of query row q (of sequence b) for indexer head gh; its
  // query heads are q/out rows sel_row * H .. + H - 1
  auto sel_row = [&](int q) { return ((int64_t)b * a.num_q + q) * a.idx_heads + gh; };

  // ---- this wave's M-tiles: tile m = kTPW*wave + j is row m / HT, head tile m % HT
  bool tvalid[kTPW];
  int trow[kTPW];
  bf16x8 qf[kTPW][4];
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const int m = kTPW * wave + j;
    const int rl = m / HT, ht = m % HT;
    tvalid[j] = rl < nrows;
    trow[j] = tvalid[j] ? rl : 0;
    const int h = ht * 16 + c;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tvalid[j] && h < H)
        v = *reinterpret_cast<const u32x4*>(
            a.q + (sel_row(q0 + rl) * H + h) * kHeadDim + kk * 32 + g * 8);
      qf[j][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // acc[j][8]: the sums of the bf16-rounded weights, formed by the same MFMAs
  // with an all-ones A operand (every entry holds the column's sum)
  f32x4 acc[kTPW][9];
  float m_run[kTPW], e_run[kTPW];
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
#pragma unroll
    for (int dt = 0; dt < 9; ++dt) acc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[j] = -INFINITY;
    e_run[j] = 0.f;
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const float scale_log2 = a.scale * kLog2eP;
  // the group's n-th page into LDS buffer bf
  const PageOffsets<PW> po(tid);
  auto load_page = [&](int n, int bf) {
    const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(L.ppid[n]) * kBlockSize * kHeadDim;
    load_page_k<PW>(a.k_cache + off, L.k[bf], po);
    load_page_v<PW>(a.v_cache + off, L.v[bf], po);
  };

  // S^T for 64 keys (kh = key subtile of 16) x the wave's M-tiles, from K in LDS
  // The products start from the page's bias (0 for a key the row selected,
  // -inf otherwise) instead of zero, so that they come out masked: a selected
  // key's score is exactly that of a zero start, any other key's is -inf.
  auto scores = [&](const uint16_t* Kl, f32x4 (&s)[4][kTPW]) {
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) {
      bf16x8 kf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kf[kk] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Kl + k_lds_index(16 * kh + c, 4 * kk + g)));
#pragma unroll
      for (int j = 0; j < kTPW; ++j) {
        f32x4 x = *reinterpret_cast<const f32x4*>(&L.bias[wave][j][16 * kh + 4 * g]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[j][kk], x, 0, 0, 0);
        s[kh][j] = x;
      }
    }
  };
  // The per-page softmax and aggregation in parts:
  //   page_max  the page maximum of the (masked) scores;
  //   reference the reference point m of the exponentials, moved rarely;
  //   weights   P = exp2(S scale - m), rounded to bf16, packed as P^T fragments;
  //   av        O^T += V^T P^T.
  auto page_max = [&](const f32x4 (&s)[4][kTPW], float (&tmax)[kTPW]) {
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      float t = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < 4; ++kh)
#pragma unroll
        for (int i = 0; i < 4; ++i) t = fmaxf(t, s[kh][j][i]);
      tmax[j] = max_over_rows(t);
    }
  };
  // the bias rows of the wave's own M-tiles for logical page pg (lane = key),
  // in the wave's own LDS rows: only this wave reads them, and its LDS
  // operations complete in order, so writing the next page's rows after this
  // page's score MFMAs have read them needs neither a barrier nor a second buffer
  auto build_bias = [&](int pg) {
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const uint64_t w = L.mask[trow[j] * kPrefillMaskPages + pg];
      L.bias[wave][j][lane] = ((w >> lane) & 1ull) ? 0.f : -INFINITY;
    }
  };
  // The reference point of the exponentials (log2 units) moves only when the
  // page's maximum exceeds it by more than kSlack; the weights then stay below
  // 2^kSlack, and numerator and denominator share the reference, so the result
  // is unchanged while most pages skip the rescale. reference() finds the new
  // point; rescale(), taken only when some lane's point moved, brings the state
  // gathered so far to it.
  auto reference = [&](const float (&tmax)[kTPW], float (&m_new)[kTPW]) {
    bool any = false;
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const float t2 = tmax[j] * scale_log2;
      const bool move = t2 > m_run[j] + kSlack;
      any |= move;
      m_new[j] = move ? t2 : m_run[j];
    }
    return any;
  };
  auto rescale = [&](const float (&m_new)[kTPW]) {
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const float alpha = m_new[j] > m_run[j]
                              ? (m_run[j] == -INFINITY ? 0.f : fast_exp2(m_run[j] - m_new[j]))
                              : 1.f;
      if constexpr (LSE) e_run[j] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 9; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][dt][i] *= alpha;
    }
  };
  // chunk ch = key subtiles 2ch, 2ch+1: keys 4g+i of each, as the V^T rows hold them
  auto weights = [&](const f32x4 (&s)[4][kTPW], const float (&m_ref)[kTPW], u32x4 (&pw)[kTPW][2],
                     float (&esum)[kTPW]) {
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
      const float m_use = m_ref[j] == -INFINITY ? 0.f : m_ref[j];
      float e = 0.f;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        uint32_t wd[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float p0 = fast_exp2(fmaf(s[2 * ch + hh][j][i], scale_log2, -m_use));
            const float p1 = fast_exp2(fmaf(s[2 * ch + hh][j][i + 1], scale_log2, -m_use));
            if constexpr (LSE) e += p0 + p1;
            wd[2 * hh + i / 2] = bf16x2_bits(p0, p1);
          }
        pw[j][ch] = u32x4{wd[0], wd[1], wd[2], wd[3]};
      }
      esum[j] = e;
    }
  };
  // O^T += V^T P^T over the two 32-key chunks. The A fragment of lane (c, g)
  // is dim 16dt + c at keys 4g .. 4g+3 and 16+4g .. 16+4g+3 of the chunk (the
  // P^T fragments' key order); two transposing reads gather it from the
  // key-major rows: in each 16-lane group, lane 4a' + b' receives element b' of
  // the 8-byte pieces that lanes a', a'+4, a'+8, a'+12 address, so lane
  // x = 4i + a' of group g addresses key 4g + i (then 16 + 4g + i), dims
  // 16dt + 4a' .. +3.
  const int vbase = (4 * g + (c >> 2)) * kVPitch + 4 * (c & 3);
  auto av = [&](const u32x4 (&pw)[kTPW][2], const uint16_t* vb) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        const uint16_t* p = vb + vbase + 32 * ch * kVPitch + 16 * dt;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(p + 16 * kVPitch));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < kTPW; ++j)
          acc[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              va, __builtin_bit_cast(bf16x8, pw[j][ch]), acc[j][dt], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kTPW; ++j)
        acc[j][8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            ones, __builtin_bit_cast(bf16x8, pw[j][ch]), acc[j][8], 0, 0, 0);
    }
  };

  // the softmax of one page's (masked) scores, then O^T += V^T P^T. Both MFMA
  // phases of a page (scores at wave priority 1, V.P at 2) run at raised
  // priority, so that the SIMD's other wave, in its softmax, yields the issue
  // slot to them (3% faster at prefill_8k than raising the V.P phase alone;
  // which of the two phases ranks higher does not matter).
  auto aggregate = [&](const f32x4 (&s)[4][kTPW], const uint16_t* vb) {
    float tmax[kTPW], m_new[kTPW], esum[kTPW];
    u32x4 pw[kTPW][2];
    page_max(s, tmax);
    if (__ballot(reference(tmax, m_new))) rescale(m_new);
#pragma unroll
    for (int j = 0; j < kTPW; ++j) m_run[j] = m_new[j];
    weights(s, m_run, pw, esum);
    if constexpr (LSE) {
#pragma unroll
      for (int j = 0; j < kTPW; ++j) e_run[j] += esum[j];
    }
    __builtin_amdgcn_s_setprio(2);
    av(pw, vb);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- the context in windows of kPrefillMaskPages pages: each window's
  // bitmask is built from the index lists, and its selected pages are streamed;
  // the softmax state carries over from window to window. The first window's
  // scan also finds the highest page any list names, which bounds the windows.
  // (WIN false: the launcher guarantees a single window, max_pages <= kPrefillMaskPages.)
  for (int w0 = 0; w0 < (WIN ? a.max_pages : 1); w0 += kPrefillMaskPages) {
    // ---- the bitmask of the group's rows, built from their index lists
    for (int i = tid; i < kRows * kPrefillMaskPages; i += kPT) L.mask[i] = 0ull;
    if (w0 == 0 && tid == 0) L.max_page = -1;
    __syncthreads();
    {
      // thread t ORs the bits of entries [8t', 8t'+8) of each row into words it
      // flushes once per page it touches (the lists are ascending)
      constexpr int E = 8;
      const int per_row = (a.topk + E - 1) / E;
      for (int job = tid; job < nrows * per_row; job += kPT) {
        const int rl = job / per_row, e0 = (job % per_row) * E;
        const int32_t* ir = a.idx + sel_row(q0 + rl) * a.topk;
        int32_t pv[E];
#pragma unroll
        for (int u = 0; u < E; ++u) pv[u] = e0 + u < a.topk ? ir[e0 + u] : -1;
        int cur = -1, top = -1;
        uint64_t word = 0ull;
#pragma unroll
        for (int u = 0; u < E; ++u) {
          const int pos = pv[u];
          if (pos < 0 || pos >= cap) continue;
          const int pg = (pos >> 6) - w0;  // page within the window
          if constexpr (WIN) {
            top = max(top, pg);
            if (pg < 0 || pg >= kPrefillMaskPages) continue;
          }
          if (pg != cur) {
            if (cur >= 0) atomicOr(&L.mask[rl * kPrefillMaskPages + cur], word);
            cur = pg;
            word = 0ull;
          }
          word |= 1ull << (pos & 63);
        }
        if (cur >= 0) atomicOr(&L.mask[rl * kPrefillMaskPages + cur], word);
        if (WIN && w0 == 0 && top >= 0) atomicMax(&L.max_page, top);
      }
    }
    __syncthreads();
    // ---- the pages that any row of the group selected, ascending, with their
    // physical ids (clamped into the pool): thread t looks at page t
    const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
    int np = 0;
    {
      const int pg = tid;  // page w0 + tid (threads beyond the window look at none)
      bool any = false;
      if (pg < kPrefillMaskPages && w0 + pg < a.max_pages)
        for (int rl = 0; rl < nrows; ++rl) any |= L.mask[rl * kPrefillMaskPages + pg] != 0ull;
      const uint64_t bal = __ballot(any);
      if (lane == 0 && wave < kPrefillMaskPages / 64) L.wcount[wave] = __popcll(bal);
      __syncthreads();
      int before = 0;
#pragma unroll
      for (int w = 0; w < kPrefillMaskPages / 64; ++w) {
        const int cw = L.wcount[w];
        before += w < wave ? cw : 0;
        np += cw;
      }
      if (any) {
        const int at = before + lanes_below(bal);
        int pid = pt[w0 + pg];
        pid = pid < 0 ? 0 : (pid >= a.num_phys ? a.num_phys - 1 : pid);
        L.plist[at] = (int16_t)pg;
        L.ppid[at] = pid;
      }
      np = __builtin_amdgcn_readfirstlane(np);
    }
    __syncthreads();

    // Every wave runs step n as scores(n) -> softmax(n) -> O += V(n) P(n);
    // page n+1's K/V rows are in flight into LDS during step n (K and V
    // double-buffered), and each wave writes its bias rows for page n+1 after
    // its score MFMAs of page n.
    if (np > 0) {
      load_page(0, 0);
      build_bias(L.plist[0]);
    }
    // The query fragments are complete before the loop on every path, and every
    // wave waits for its direct page loads before the barrier that publishes
    // the page.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int n = 0, bf = 0; n < np; ++n, bf ^= 1) {
      const bool more = n + 1 < np;
      if (more) load_page(n + 1, bf ^ 1);  // in flight during this page
      f32x4 sc[4][kTPW];
      __builtin_amdgcn_s_setprio(1);
      scores(L.k[bf], sc);
      __builtin_amdgcn_s_setprio(0);
      if (more) build_bias(L.plist[n + 1]);
      aggregate(sc, L.v[bf]);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
      __syncthreads();  // page n+1 stored; the buffers of page n free
    }
    if (!WIN || L.max_page < w0 + kPrefillMaskPages) break;  // block-uniform (after barriers)
    __syncthreads();  // every wave is done with this window's mask and pages
  }

  // ---- outputs: lanes c, c+16, c+32, c+48 hold disjoint key sets
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const float l = acc[j][8][0];
    // the fp32 sum of the weights serves the log-sum-exp only, and is kept
    // only when the caller asks for it
    const float e = LSE ? sum_over_rows(e_run[j]) : 0.f;
    const int m = kTPW * wave + j;
    const int ht = m % HT, h = ht * 16 + c;
    if (!tvalid[j] || h >= H) continue;
    const int64_t rowq = sel_row(q0 + trow[j]);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    uint16_t* orow = a.out + (rowq * H + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      u32x2 pk;
      pk.x = f32_to_bf16_bits(acc[j][dt][0] * inv) | (f32_to_bf16_bits(acc[j][dt][1] * inv) << 16);
      pk.y = f32_to_bf16_bits(acc[j][dt][2] * inv) | (f32_to_bf16_bits(acc[j][dt][3] * inv) << 16);
      *reinterpret_cast<u32x2*>(orow + dt * 16 + g * 4) = pk;
    }
    if (LSE && g == 0)
      a.lse[rowq * H + h] = e > 0.f ? (m_run[j] + fast_log2(e)) * kLn2P : -INFINITY;
  }
}

// The mask-scheduled kernel computes every key of each page any row of its
// group selected, the per-row gather only the selected keys; per key the
// former costs about a quarter of the latter (2048-row chunks at topk 2048:
// 441 us over 16K-position rows against 245 us for the gather), so it is
// chosen while a row's context averages at most 4 x topk positions. The rows
// are taken to end at the longest context (a prefill chunk, or the whole
// prompt): their average context is that length less half their count.
// Contexts above kPrefillMaskPages pages are walked in windows of that many.
bool prefill_attend_supported(int max_pages, int num_q, int num_heads, int topk) {
  const int64_t cap = (int64_t)max_pages * kBlockSize;
  const int64_t avg = cap - (num_q < cap ? num_q : cap) / 2;
  return num_heads <= 64 && avg <= (int64_t)4 * topk;
}


hipError_t launch_prefill_attend(const AttendArgs& a, int batch, hipStream_t s) {
  constexpr int PW = 4;
  const int ht = (a.num_heads + 15) / 16;
  const int qb = PW * kTPW / ht;
  const int64_t blocks = (int64_t)batch * a.idx_heads * ((a.num_q + qb - 1) / qb);
  dim3 grid((unsigned)blocks);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(64 * PW), 0, s, a); };
  const bool lse = a.lse != nullptr;
  auto pick = [&](auto win) {
    constexpr bool W = decltype(win)::value;
    if (ht == 1)
      lse ? go(prefill_attend_kernel<1, PW, true, W>) : go(prefill_attend_kernel<1, PW, false, W>);
    else if (ht == 2)
      lse ? go(prefill_attend_kernel<2, PW, true, W>) : go(prefill_attend_kernel<2, PW, false, W>);
    else if (ht == 3)
      lse ? go(prefill_attend_kernel<3, PW, true, W>) : go(prefill_attend_kernel<3, PW, false, W>);
    else
      lse ? go(prefill_attend_kernel<4, PW, true, W>) : go(prefill_attend_kernel<4, PW, false, W>);
  };
  if (a.max_pages > kPrefillMaskPages) pick(std::true_type{});
  else pick(std::false_type{});
  return hipGetLastError();
}

}  // namespace tis
