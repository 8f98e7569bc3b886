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
// dimension. One wave handles one (row, split) for all heads, 32 keys per tile:
//   S^T = K . Q^T   bf16 MFMA 16x16x32, keys x heads, fp32 accumulate;
//   online softmax per head in fp32 (base-2 exponent, running max and sum);
//   O^T += V^T . P^T with P rounded to bf16 (its rounded values also form the
//   running sum, so the output is an exact convex combination of V rows);
//   V^T goes through LDS, transposed while it is stored.
// With the keys-by-heads layout every lane keeps the statistics, the P^T
// fragment and the O^T columns of one head, so no cross-lane shuffles are
// needed to rescale the accumulators.
//
// Decode ("Separate Paths for Prefill and Decode": memory-bound, index
// prefetch overlapped with incremental aggregation) splits a row's selection
// over several waves and merges their partial (max, sum, accumulator) states in
// `combine`. Within a wave the indices and page ids of tile t+1 are fetched
// while tile t is being aggregated. Prefill (compute-bound, many rows) gives
// each row one wave and writes the result directly.
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

// Online-softmax state of the HT head tiles a lane works on.
template <int HT>
struct AttendState {
  bf16x8 qf[HT][4];  // Q^T fragments (MFMA B operand): head 16*ht + c, dims 32*kk + 8*g
  f32x4 acc[8][HT];  // O^T: dims 16*dt + 4*g + i of head 16*ht + c
  float m_run[HT], l_run[HT], e_run[HT];
};

// Aggregate one tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
template <int HT>
__device__ __forceinline__ void attend_tile(AttendState<HT>& st, const KvTile& t, uint16_t* vt,
                                            float scale_log2, int lane) {
  const int c = lane & 15, g = lane >> 4;
  f32x4 s[2][HT];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.kf[kh][kk], st.qf[ht][kk], x, 0, 0, 0);
      s[kh][ht] = x;
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

  // online softmax; lane owns head 16*ht + c and keys {4g+i, 16+4g+i}
  u32x4 pw[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    float v[8];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kh * 16 + g * 4 + i;
        v[kh * 4 + i] = ((t.vmask >> key) & 1ull) ? s[kh][ht][i] * scale_log2 : -INFINITY;
      }
    float tmax = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, v[e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(st.m_run[ht], tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(st.m_run[ht] - m_use);
    st.m_run[ht] = m_new;
    float lsum = 0.f, esum = 0.f;
    uint32_t pb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = fast_exp2(v[e] - m_use);
      pb[e] = f32_to_bf16_bits(pe);
      lsum += __uint_as_float(pb[e] << 16);
      esum += pe;
    }
    st.l_run[ht] = st.l_run[ht] * alpha + lsum;
    st.e_run[ht] = st.e_run[ht] * alpha + esum;
    pw[ht] = u32x4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                   pb[6] | (pb[7] << 16)};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acc[dt][ht] *= alpha;
  }

  __syncthreads();  // vt stores are visible
  // O^T += V^T P^T
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint16_t* vrow = &vt[(dt * 16 + c) * kVtStride];
    const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + g * 4);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 + g * 4);
    const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
      st.acc[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          va, __builtin_bit_cast(bf16x8, pw[ht]), st.acc[dt][ht], 0, 0, 0);
  }
}

// HT head tiles of 16 per wave. The indices and page ids of tile t+1 are
// fetched while tile t is aggregated. (Holding a second K/V tile in registers
// to overlap its gather as well was measured slower: it halves the waves that
// fit on a SIMD.)
template <int HT>
__global__ __launch_bounds__(64) void attend_kernel(AttendArgs a) {
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
  const int b = r / a.num_q;
  const int lane = threadIdx.x;
  const int c = lane & 15, g = lane >> 4;
  const int H = a.num_heads;
  const int64_t cap = (int64_t)a.max_pages * kBlockSize;
  const int k_begin = sp * a.keys_per_split;
  const int k_end = min(k_begin + a.keys_per_split, a.topk);
  const int32_t* idxr = a.idx + (int64_t)r * a.topk;
  const float scale_log2 = a.scale * kLog2e;

  AttendState<HT> st;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = (hg * HT + ht) * 16 + c;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < H)
        v = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)r * H + h) * kHeadDim + kk * 32 + g * 8);
      st.qf[ht][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) st.acc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  // l_run: sum of the bf16-rounded weights (normalises the output, so that it
  // is an exact convex combination of V rows); e_run: fp32 sum for the lse
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    st.m_run[ht] = -INFINITY;
    st.l_run[ht] = 0.f;
    st.e_run[ht] = 0.f;
  }

  // index -> physical row of the tile at t0 (lanes 0..31 hold one key each)
  auto fetch_rows = [&](int t0, int64_t* row, bool* ok) {
    int pos = -1;
    if (lane < 32 && t0 + lane < k_end) pos = idxr[t0 + lane];
    *ok = pos >= 0 && pos < cap;
    *row = *ok ? phys_row(a.page_table, b, a.max_pages, a.num_phys, pos) : 0;
  };

  constexpr int T = kAttendTile;
  if (k_begin < k_end) {
    int64_t row;
    bool ok;
    fetch_rows(k_begin, &row, &ok);
    KvTile ta;
    for (int t0 = k_begin; t0 < k_end; t0 += T) {
      load_tile(ta, a, row, ok, lane);
      // prefetch the next tile's indices and page ids
      if (t0 + T < k_end) fetch_rows(t0 + T, &row, &ok);
      attend_tile<HT>(st, ta, vt, scale_log2, lane);
    }
  }
  float* m_run = st.m_run;
  float* l_run = st.l_run;
  float* e_run = st.e_run;
  auto& acc = st.acc;

  // totals per head: lanes c, c+16, c+32, c+48 hold disjoint key sets
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    l_run[ht] += __shfl_xor(l_run[ht], 16);
    l_run[ht] += __shfl_xor(l_run[ht], 32);
    e_run[ht] += __shfl_xor(e_run[ht], 16);
    e_run[ht] += __shfl_xor(e_run[ht], 32);
  }

  if (a.n_splits == 1) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = (hg * HT + ht) * 16 + c;
      if (h >= H) continue;
      const float inv = l_run[ht] > 0.f ? 1.0f / l_run[ht] : 0.f;
      uint16_t* orow = a.out + ((int64_t)r * H + h) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          orow[dt * 16 + g * 4 + i] = (uint16_t)f32_to_bf16_bits(acc[dt][ht][i] * inv);
      if (a.lse && g == 0)
        a.lse[(int64_t)r * H + h] =
            e_run[ht] > 0.f ? (m_run[ht] + fast_log2(e_run[ht])) * kLn2 : -INFINITY;
    }
  } else {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = (hg * HT + ht) * 16 + c;
      if (h >= H) continue;
      float* prow = a.part_o + ((int64_t)unit * H + h) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) prow[dt * 16 + g * 4 + i] = acc[dt][ht][i];
      if (g == 0) {
        a.part_ml[((int64_t)unit * H + h) * 3 + 0] = m_run[ht];
        a.part_ml[((int64_t)unit * H + h) * 3 + 1] = l_run[ht];
        a.part_ml[((int64_t)unit * H + h) * 3 + 2] = e_run[ht];
      }
    }
  }
}

// Merge the split states of one (row, head) with 256 threads. The split
// statistics are read one split per thread (n_splits <= 256) and reduced over
// the block; thread t then accumulates channels 2*(t % 64) and 2*(t % 64) + 1
// over the splits t / 64, t / 64 + 4, ..., with eight splits' loads issued
// before any is used, and the four partial sums meet in LDS. Every sum runs in
// a fixed order, so the result is deterministic.
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
  float M = wave_max(m);
  if (lane == 0) s_red[0][grp] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
  if (tid < ns) s_f[tid] = f;
  float L = l * f, E = e * f;
  for (int o = 32; o >= 1; o >>= 1) {
    L += __shfl_xor(L, o);
    E += __shfl_xor(E, o);
  }
  if (lane == 0) {
    s_red[1][grp] = L;
    s_red[2][grp] = E;
  }
  __syncthreads();
  L = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  E = (s_red[2][0] + s_red[2][1]) + (s_red[2][2] + s_red[2][3]);

  float o0 = 0.f, o1 = 0.f;
  constexpr int U = 8;
  for (int s0 = grp; s0 < ns; s0 += 4 * U) {
    float2 po[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + 4 * u;
      po[u] = sp < ns ? *reinterpret_cast<const float2*>(a.part_o + ((u0 + sp) * H + h) * kHeadDim +
                                                          2 * lane)
                      : float2{0.f, 0.f};
    }
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
    const uint32_t packed = f32_to_bf16_bits(o0 * inv) | (f32_to_bf16_bits(o1 * inv) << 16);
    *reinterpret_cast<uint32_t*>(orow + 2 * lane) = packed;
    if (a.lse && lane == 0)
      a.lse[(int64_t)r * H + h] = E > 0.f ? (M + fast_log2(E)) * kLn2 : -INFINITY;
  }
}

#ifndef TIS_ATTEND_HEAD_TILES
#define TIS_ATTEND_HEAD_TILES 1  // 16-head tiles per wave
#endif

hipError_t launch_attend(const AttendArgs& a0, hipStream_t s) {
  AttendArgs a = a0;
  const int tiles = (a.num_heads + 15) / 16;
  const int ht = tiles < TIS_ATTEND_HEAD_TILES ? tiles : TIS_ATTEND_HEAD_TILES;
  a.head_groups = (tiles + ht - 1) / ht;
  const int64_t units = (int64_t)a.rows * a.n_splits;
  const int64_t blocks =
      a.head_groups == 1 ? units : (units + 7) / 8 * 8 * a.head_groups;
  dim3 grid((unsigned)blocks);
  if (ht == 1)
    hipLaunchKernelGGL((attend_kernel<1>), grid, dim3(64), 0, s, a);
  else if (ht == 2)
    hipLaunchKernelGGL((attend_kernel<2>), grid, dim3(64), 0, s, a);
  else if (ht == 3)
    hipLaunchKernelGGL((attend_kernel<3>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((attend_kernel<4>), grid, dim3(64), 0, s, a);
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
