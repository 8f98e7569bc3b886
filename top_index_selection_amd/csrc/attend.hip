// attend.hip -- paged gather + exact sparse attention for gfx950.
//
// For every query row, the K and V rows of the selected positions are fetched
// through the page table ("Day-0 Inference Adaptation of Ultra-Large-Scale MoE
// Models on Domestic AI Accelerators", section 4.1, step 3: gather full KV by
// indices and perform exact attention; "Day-0 Adaptation for Trillion-Parameter
// MoE Models", section IV: gather the selected pages, then a prefill or a
// decode kernel) and a softmax over exactly those positions is applied.
//
// All H query heads of a row share one K/V head, so the heads form one MFMA
// dimension. One wave handles one (row, split) for 16 of the heads, 32 keys per
// tile:
//   S^T = K . Q^T   bf16 MFMA 16x16x32, keys x heads, fp32 accumulate;
//   online softmax per head in fp32 (base-2 exponent);
//   O^T += V^T . P^T with P rounded to bf16; an all-ones A operand sums the
//   rounded weights in the same MFMA pass, and that sum normalises the output,
//   so the output is an exact convex combination of V rows;
//   V^T goes through LDS, transposed while it is stored.
// With the keys-by-heads layout every lane keeps the statistics, the P^T
// fragment and the O^T columns of one head, so no cross-lane shuffles are
// needed to rescale the accumulators.
//
// Decode ("Separate Paths for Prefill and Decode": memory-bound, index
// prefetch overlapped with incremental aggregation) splits a row's selection
// over several waves and merges their partial (reference, sums, accumulator)
// states in `combine`. Within a wave the indices and page ids of a chunk of
// tiles are fetched first, and the K/V rows of tile t+1 are in flight while
// tile t is aggregated. With a single split per row (paged_gather_attend in
// the decode phase on enough rows), a wave writes the result directly.
#include "tis_common.h"
#include "tis_internal.h"

namespace tis {

constexpr int kVtStride = 36;  // LDS row pitch of V^T in bf16 (32 keys + 4 pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;


// The gathered K and V rows of one 32-key tile, held in registers: K as MFMA
// A fragments (key kh*16 + c, dims 32*kk + 8*g), V as 4 keys x 8 dims per lane
// and rep, plus the mask of keys that hold a valid position.
struct KvTile {
  bf16x8 kf[2][4];
  u32x4 vv[2][4];
  uint64_t vmask;
};

__device__ __forceinline__ void load_tile(KvTile& t, const AttendArgs& a, int64_t row, bool ok,
                                          int lane) {
  const int c = lane & 15, g = lane >> 4;
  t.vmask = __ballot(ok) & 0xffffffffull;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int64_t rk = __shfl(row, kh * 16 + c);
    const uint16_t* kr = a.k_cache + rk * kHeadDim + g * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      t.kf[kh][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + kk * 32));
  }
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int bi = lane + 64 * rep;
    const int kq = bi & 7, dc = bi >> 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t rv = __shfl(row, kq * 4 + e);
      t.vv[rep][e] = *reinterpret_cast<const u32x4*>(a.v_cache + rv * kHeadDim + dc * 8);
    }
  }
}

// Online-softmax state of the lane's head (16 heads per wave, head c of the tile).
struct AttendState {
  bf16x8 qf[4];  // Q^T fragments (MFMA B operand): head c, dims 32*kk + 8*g
  f32x4 acc[8];  // O^T: dims 16*dt + 4*g + i of head c
  f32x4 accl;    // sum of the bf16-rounded weights (every entry holds the head's sum)
  float m_run;   // reference point of the exponentials (log2 units)
  float e_run;   // fp32 sum of the weights over the lane's keys (for the lse)
};

constexpr float kSlack = 8.0f;  // log2 headroom of the softmax weights

// Aggregate one tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
__device__ __forceinline__ void attend_tile(AttendState& st, const KvTile& t, uint16_t* vt,
                                            float scale_log2, bf16x8 ones, int lane) {
  const int c = lane & 15, g = lane >> 4;
  f32x4 s[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.kf[kh][kk], st.qf[kk], x, 0, 0, 0);
    s[kh] = x;
  }

  // V^T into LDS (4 keys x 8 dims per lane and rep, stored as 8 rows of 4 keys)
  __syncthreads();  // previous tile's reads of vt are done
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int bi = lane + 64 * rep;
    const int kq = bi & 7, dc = bi >> 3;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x0 = t.vv[rep][0][w], x1 = t.vv[rep][1][w], x2 = t.vv[rep][2][w],
                     x3 = t.vv[rep][3][w];
      u32x2 lo, hi;
      lo.x = (x0 & 0xffffu) | (x1 << 16);
      lo.y = (x2 & 0xffffu) | (x3 << 16);
      hi.x = (x0 >> 16) | (x1 & 0xffff0000u);
      hi.y = (x2 >> 16) | (x3 & 0xffff0000u);
      *reinterpret_cast<u32x2*>(&vt[(dc * 8 + 2 * w) * kVtStride + kq * 4]) = lo;
      *reinterpret_cast<u32x2*>(&vt[(dc * 8 + 2 * w + 1) * kVtStride + kq * 4]) = hi;
    }
  }

  // Online softmax; the lane owns head c and keys 16kh + 4g + i. Keys without a
  // valid position become -inf: key 16kh + 4g + i is bit 16kh + i of the valid
  // mask shifted down by 4g, and a sign-extended one-bit field selects between
  // the score's bits and those of -inf.
  const uint32_t wv = (uint32_t)t.vmask >> (4 * g);
  float v[8];
  float tmax = -INFINITY;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)wv, 16 * kh + i, 1);
      v[kh * 4 + i] = __uint_as_float((__float_as_uint(s[kh][i]) & m) | (0xff800000u & ~m));
      tmax = fmaxf(tmax, v[kh * 4 + i]);
    }
  tmax = max_over_rows(tmax);
  // The reference point moves only when the tile's maximum exceeds it by more
  // than kSlack: the weights then stay below 2^kSlack, and numerator and
  // denominators share the reference, so the result does not depend on it.
  const float t2 = tmax * scale_log2;
  const bool move = t2 > st.m_run + kSlack;
  if (__ballot(move)) {
    const float m_new = move ? t2 : st.m_run;
    const float alpha = st.m_run == -INFINITY ? 0.f : fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
    st.e_run *= alpha;
    st.accl *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acc[dt] *= alpha;
  }
  const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
  float esum = 0.f;
  uint32_t pw[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float p0 = fast_exp2(fmaf(v[e], scale_log2, -m_use));
    const float p1 = fast_exp2(fmaf(v[e + 1], scale_log2, -m_use));
    pw[e / 2] = bf16x2_bits(p0, p1);
    esum += p0 + p1;
  }
  st.e_run += esum;
  const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});

  __syncthreads();  // vt stores are visible
  // O^T += V^T P^T, and the weight sums through an all-ones A operand
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint16_t* vrow = &vt[(dt * 16 + c) * kVtStride];
    const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + g * 4);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 + g * 4);
    const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, st.acc[dt], 0, 0, 0);
  }
  st.accl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, st.accl, 0, 0, 0);
}

// One wave per (row, split, 16-head tile). A split is walked in chunks of
// kChunk tiles: the chunk's indices are loaded, then its page ids, all in
// flight together; then the K/V rows of tile j+1 are in flight while tile j is
// aggregated (two tiles of registers, which fit two waves per SIMD).
constexpr int kChunk = 4;

__global__ __launch_bounds__(64, 2) void attend_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kHeadDim * kVtStride];

  // The head groups of one (row, split) unit are 8 blocks apart: blocks are
  // handed to the 8 XCDs in turn, so they run on one XCD and share its L2 copy
  // of the gathered K/V rows.
  int unit = blockIdx.x, hg = 0;
  if (a.head_groups > 1) {
    const int span = 8 * a.head_groups;
    hg = (int)(blockIdx.x % span) / 8;
    unit = (int)(blockIdx.x / span) * 8 + (int)(blockIdx.x % 8);
    if (unit >= a.rows * a.n_splits) return;  // padding of the last group of 8
  }
  const int r = unit / a.n_splits, sp = unit % a.n_splits;
  const int b = r / (a.num_q * a.idx_heads);  // selection row r's sequence
  const int lane = threadIdx.x;
  const int c = lane & 15, g = lane >> 4;
  const int H = a.num_heads;
  const int h = hg * 16 + c;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int k_begin = sp * a.keys_per_split;
  const int k_end = min(k_begin + a.keys_per_split, a.topk);
  const int32_t* idxr = a.idx + (int64_t)r * a.topk;
  const int32_t* ptb = a.page_table + (int64_t)b * a.max_pages;
  const float scale_log2 = a.scale * kLog2e;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  AttendState st;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (h < H)
      v = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)r * H + h) * kHeadDim + kk * 32 + g * 8);
    st.qf[kk] = __builtin_bit_cast(bf16x8, v);
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.accl = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.e_run = 0.f;

  constexpr int T = kAttendTile;
  for (int c0 = k_begin; c0 < k_end; c0 += kChunk * T) {
    // indices of the chunk's tiles (lane l and l + 32 both hold key l of a tile)
    int pos[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int e = c0 + j * T + (lane & 31);
      const int v = idxr[min(e, k_end - 1)];
      pos[j] = e < k_end ? v : -1;
    }
    // their physical rows (page ids clamped into the pool)
    int64_t row[kChunk];
    bool ok[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      ok[j] = pos[j] >= 0 && pos[j] < cap;
      int pg = pos[j] >> 6;
      pg = pg < 0 ? 0 : (pg >= a.max_pages ? a.max_pages - 1 : pg);
      int pid = ptb[pg];
      pid = pid < 0 ? 0 : (pid >= a.num_phys ? a.num_phys - 1 : pid);
      row[j] = ok[j] ? (int64_t)pid * kBlockSize + (pos[j] & (kBlockSize - 1)) : 0;
    }
    // Every row of the chunk is resolved here, before the first tile's loads
    // are issued: otherwise the compiler moves a later tile's page-id load
    // into the branch that uses it, behind the first tile's loads, and the
    // in-order wait counter then drains those before the next tile is issued.
    // (An empty statement: it only pins where the values are computed.)
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      asm volatile("" ::"v"((uint32_t)row[j]), "v"((uint32_t)(row[j] >> 32)));
    KvTile tt[2];
    load_tile(tt[0], a, row[0], ok[0], lane);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (c0 + j * T >= k_end) break;
      if (j + 1 < kChunk && c0 + (j + 1) * T < k_end)
        load_tile(tt[(j + 1) & 1], a, row[j + 1], ok[j + 1], lane);
      attend_tile(st, tt[j & 1], vt, scale_log2, ones, lane);
    }
  }

  // totals per head: lanes c, c+16, c+32, c+48 hold disjoint key sets of e_run;
  // accl already sums over all keys
  const float l_run = st.accl[0];
  const float e_run = sum_over_rows(st.e_run);
  if (h >= H) return;

  if (a.n_splits == 1) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    uint16_t* orow = a.out + ((int64_t)r * H + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      u32x2 pk;
      pk.x = bf16x2_bits(st.acc[dt][0] * inv, st.acc[dt][1] * inv);
      pk.y = bf16x2_bits(st.acc[dt][2] * inv, st.acc[dt][3] * inv);
      *reinterpret_cast<u32x2*>(orow + dt * 16 + g * 4) = pk;
    }
    if (a.lse && g == 0)
      a.lse[(int64_t)r * H + h] = e_run > 0.f ? (st.m_run + fast_log2(e_run)) * kLn2 : -INFINITY;
  } else {
    float* prow = a.part_o + ((int64_t)unit * H + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(prow + dt * 16 + g * 4) = st.acc[dt];
    if (g == 0) {
      a.part_ml[((int64_t)unit * H + h) * 3 + 0] = st.m_run;
      a.part_ml[((int64_t)unit * H + h) * 3 + 1] = l_run;
      a.part_ml[((int64_t)unit * H + h) * 3 + 2] = e_run;
    }
  }
}

// Merge the split states of one (row, head) with 256 threads. The split
// statistics are read one split per thread (n_splits <= 256), and right after
// them the first partial outputs, so that those loads are in flight while the
// statistics are reduced over the block. Thread t accumulates channels
// 2*(t % 64) and 2*(t % 64) + 1 over the splits t / 64, t / 64 + 4, ..., eight
// splits' loads at a time, and the four partial sums meet in LDS. Every sum
// runs in a fixed order, so the result is deterministic.
__global__ __launch_bounds__(256) void combine_kernel(AttendArgs a) {
  __shared__ float s_f[kMaxSplits];
  __shared__ float s_red[3][4];
  __shared__ float2 s_o[3][64];
  const int r = blockIdx.x / a.num_heads, h = blockIdx.x % a.num_heads;
  const int tid = threadIdx.x, lane = tid & 63, grp = tid >> 6;
  const int H = a.num_heads, ns = a.n_splits;
  const int64_t u0 = (int64_t)r * ns;

  float m = -INFINITY, l = 0.f, e = 0.f;
  if (tid < ns) {
    const float* ml = a.part_ml + ((u0 + tid) * H + h) * 3;
    m = ml[0];
    l = ml[1];
    e = ml[2];
  }
  constexpr int U = 8;
  float2 po[U];
  auto load_po = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + 4 * u;
      po[u] = sp < ns ? *reinterpret_cast<const float2*>(a.part_o + ((u0 + sp) * H + h) * kHeadDim +
                                                          2 * lane)
                      : float2{0.f, 0.f};
    }
  };
  load_po(grp);

  float M = wave_max(m);
  if (lane == 0) s_red[0][grp] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
  if (tid < ns) s_f[tid] = f;
  float L = wave_sum(l * f), E = wave_sum(e * f);
  if (lane == 0) {
    s_red[1][grp] = L;
    s_red[2][grp] = E;
  }
  __syncthreads();
  L = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  E = (s_red[2][0] + s_red[2][1]) + (s_red[2][2] + s_red[2][3]);

  float o0 = 0.f, o1 = 0.f;
  for (int s0 = grp; s0 < ns; s0 += 4 * U) {
    if (s0 != grp) load_po(s0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + 4 * u;
      const float fk = sp < ns ? s_f[sp] : 0.f;
      o0 = fmaf(po[u].x, fk, o0);
      o1 = fmaf(po[u].y, fk, o1);
    }
  }
  if (grp > 0) s_o[grp - 1][lane] = float2{o0, o1};
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      o0 += s_o[g][lane].x;
      o1 += s_o[g][lane].y;
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    uint16_t* orow = a.out + ((int64_t)r * H + h) * kHeadDim;
    *reinterpret_cast<uint32_t*>(orow + 2 * lane) = bf16x2_bits(o0 * inv, o1 * inv);
    if (a.lse && lane == 0)
      a.lse[(int64_t)r * H + h] = E > 0.f ? (M + fast_log2(E)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_attend(const AttendArgs& a0, hipStream_t s) {
  AttendArgs a = a0;
  a.head_groups = (a.num_heads + 15) / 16;
  const int64_t units = (int64_t)a.rows * a.n_splits;
  const int64_t blocks =
      a.head_groups == 1 ? units : (units + 7) / 8 * 8 * a.head_groups;
  hipLaunchKernelGGL(attend_kernel, dim3((unsigned)blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const AttendArgs& a, hipStream_t s) {
  if (a.n_splits == 1) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((int64_t)a.rows * a.num_heads)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- cache append

// One block per sequence: write the new token's rows at position seq_lens[b]
// and advance seq_lens[b]. A full cache is left unchanged.
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int64_t pos = a.seq_lens[b];
  if (pos < 0 || pos >= cap) return;
  const int64_t row = phys_row(a.page_table, b, a.max_pages, a.num_phys, pos);
  // 128 channels of K and V: two per lane; d_c channels of k_comp
  a.k_cache[row * kHeadDim + 2 * lane] = a.k_new[(int64_t)b * kHeadDim + 2 * lane];
  a.k_cache[row * kHeadDim + 2 * lane + 1] = a.k_new[(int64_t)b * kHeadDim + 2 * lane + 1];
  a.v_cache[row * kHeadDim + 2 * lane] = a.v_new[(int64_t)b * kHeadDim + 2 * lane];
  a.v_cache[row * kHeadDim + 2 * lane + 1] = a.v_new[(int64_t)b * kHeadDim + 2 * lane + 1];
  for (int ch = lane; ch < a.d_c; ch += 64)
    a.k_comp_cache[row * a.d_c + ch] = a.k_comp_new[(int64_t)b * a.d_c + ch];
  __syncthreads();
  if (lane == 0) a.seq_lens[b] = (int32_t)(pos + 1);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace tis
