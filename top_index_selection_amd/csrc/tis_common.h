// tis_common.h -- device helpers shared by the gfx950 kernels of libtis.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tis {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBlockSize = 64;   // tokens per KV page (the only supported size)
constexpr int kHeadDim = 128;    // head_dim (the only supported size)
constexpr int kHistBits = 12;    // first radix digit: sign, exponent, 3 mantissa bits
constexpr int kHistBins = 1 << kHistBits;
// A row's first-digit histogram in the workspace: the 4096 fine bins, then 64
// coarse counts, one per group of 64 consecutive bins.
constexpr int kHistGroups = kHistBins / 64;
constexpr int kRowHistWords = kHistBins + kHistGroups;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ numbers

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values -> packed bf16 pair (lo, hi), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Order-preserving map of an fp32 score to an unsigned key: a larger score gets
// a larger key, and -0.0 maps like +0.0 so that the two compare equal (ties are
// then decided by position, as for any equal scores).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Hardware base-2 exponential and logarithm (the softmax runs in base 2).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// number of set bits of a 64-bit lane mask strictly below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// DPP lane exchanges inside 16-lane rows (row_mask/bank_mask all lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor3 = 0x1B;        // quad_perm [3,2,1,0]
constexpr int kDppQuadSwapPairs = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes (xor 7)
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within 16 lanes (xor 15)

// Max and sum over the four lanes c, c+16, c+32 and c+48 of a wave, with
// gfx950's cross-row lane swaps (VALU moves, no LDS round trip): the 16-lane
// swap pairs rows 0-1 and 2-3, the 32-lane swap the two halves. The pairing is
// that of xor-16 then xor-32 shuffles, so sums come out bitwise the same.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reduction over the whole wave: within each row of 16 lanes by DPP moves
// (pairs, quads, half-row mirror, row mirror), then across rows by the lane
// swaps. Every lane receives the result.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppQuadSwapPairs>(v));
  v = op(v, dpp<kDppRowHalfMirror>(v));
  v = op(v, dpp<kDppRowMirror>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}

// Inclusive prefix sum across the wave, on DPP lane moves: within each row of
// 16 lanes, shifts right by 1, 2, 4 and 8 with zeros shifted in; then the last
// lane of row 0 (of row 2) is added to row 1 (to row 3), and the last lane of
// row 1 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// Block barrier that orders LDS accesses only: unlike __syncthreads() it does
// not wait for the wave's global loads and stores still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive prefix sum over a block of NT threads (a multiple of 64); returns
// the thread's exclusive prefix and writes the block total to *total. `tmp`
// holds NT / 64 ints of LDS. Contains __syncthreads(); every thread of the
// block must call it.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane_id() == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    int t = tmp[i];
    before += (i < w) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Adds a block's LDS histogram (kHistBins bins) into a row histogram of
// kRowHistWords words. The fine bins: a wave's additions cover 64 consecutive
// bins (two cache lines) at a time. The coarse groups: thread t sums the BPT =
// kHistBins / NT bins from BPT*t, the 64 / BPT threads of a group of 64 bins
// (consecutive lanes) add their sums by DPP moves, and the group's first thread
// adds the total. NT threads; s_hist must be complete (after a barrier).
template <int NT = 256>
__device__ __forceinline__ void add_row_hist(const uint32_t* s_hist, uint32_t* out) {
  constexpr int BPT = kHistBins / NT;  // 16 (256 threads) or 4 (1024)
  constexpr int TPG = 64 / BPT;        // threads per group: 4 or 16
  static_assert(BPT % 4 == 0 && (TPG == 4 || TPG == 16), "256 or 1024 threads");
  const int tid = threadIdx.x;
  const u32x4* q = reinterpret_cast<const u32x4*>(s_hist) + tid * (BPT / 4);
  u32x4 x[BPT / 4];
#pragma unroll
  for (int k = 0; k < BPT / 4; ++k) x[k] = q[k];
  for (int i = tid; i < kHistBins; i += NT) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(&out[i], c);
  }
  int g = 0;
#pragma unroll
  for (int k = 0; k < BPT / 4; ++k) g += (int)(x[k].x + x[k].y + x[k].z + x[k].w);
  g += __builtin_amdgcn_update_dpp(0, g, kDppXor1, 0xf, 0xf, false);
  g += __builtin_amdgcn_update_dpp(0, g, kDppQuadSwapPairs, 0xf, 0xf, false);
  if constexpr (TPG == 16) {  // quads -> halves of a 16-lane row -> the row
    g += __builtin_amdgcn_update_dpp(0, g, kDppRowHalfMirror, 0xf, 0xf, false);
    g += __builtin_amdgcn_update_dpp(0, g, kDppRowMirror, 0xf, 0xf, false);
  }
  if ((tid & (TPG - 1)) == 0 && g) atomicAdd(&out[kHistBins + tid / TPG], (uint32_t)g);
}

// ------------------------------------------------------------ addressing

// Physical row of logical position j in sequence b, with the page id clamped
// into the pool so that a bad page table cannot send an access out of bounds.
__device__ __forceinline__ int64_t phys_row(const int32_t* __restrict__ page_table, int b,
                                            int max_pages, int num_phys, int64_t j) {
  int64_t g = j >> 6;
  g = g < 0 ? 0 : (g >= max_pages ? max_pages - 1 : g);
  int pid = page_table[(int64_t)b * max_pages + g];
  pid = pid < 0 ? 0 : (pid >= num_phys ? num_phys - 1 : pid);
  return (int64_t)pid * kBlockSize + (j & (kBlockSize - 1));
}

// Query position of row i of sequence b, and the number of causal candidates.
struct RowGeom {
  int64_t p;  // query position (clamped into the cache)
  int64_t n;  // candidates 0..p, i.e. p + 1 (0 for an empty row)
};

__device__ __forceinline__ RowGeom row_geom(const int32_t* __restrict__ seq_lens,
                                            const int32_t* __restrict__ q_start, int S_q,
                                            int b, int i, int64_t cap) {
  int64_t L = seq_lens ? (int64_t)seq_lens[b] : cap;
  L = L > cap ? cap : L;
  int64_t first = q_start ? (int64_t)q_start[b] : L - S_q;
  int64_t p = first + i;
  if (p >= L) p = L - 1;
  RowGeom g;
  g.p = p;
  g.n = p >= 0 ? p + 1 : 0;
  return g;
}

}  // namespace tis
