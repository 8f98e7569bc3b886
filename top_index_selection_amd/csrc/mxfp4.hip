// mxfp4.hip -- online MXFP4 -> FP8 (E4M3) conversion of expert weights, gfx950.
//
// Expert weights stay in memory in MXFP4; when a router selects an expert,
// its weights are dequantised into an 8-bit working format just before use,
// into a working buffer that successive layers reuse ("Day-0 Inference
// Adaptation for Ultra-Large MoE Models on Domestic GPUs", section "Handling
// Low-Precision Expert Weights: Online Conversion and Workspace Reuse"; "Day-0
// Adaptation for Trillion-Parameter MoE Models", section V).
//
// Formats: OCP Microscaling (MX) v1.0 -- E2M1 elements (two per byte, element
// 2i in the low nibble of byte i) with one E8M0 scale 2^(X-127) per 32
// consecutive elements of a row, X = 255 meaning NaN -- and OCP FP8 E4M3
// (bias 7, largest finite 448, S.1111.111 NaN). An element's value
// e * 2^(X-127+offset) is rounded to nearest E4M3, ties to even; finite
// results above 448 saturate to 448; zeros and NaNs keep the element's sign.
//
// The kernel is bound by HBM bandwidth: 0.5 + 1/32 bytes read and 1 byte
// written per element. Every value an element can take is one of 8
// magnitudes times the block's scale, so a workgroup first tabulates, for all
// 256 scale bytes, the E4M3 bytes of the 8 magnitudes (two dwords per scale,
// in LDS). A lane then converts 16 elements (8 packed bytes) at a time: the
// nibbles are spread to bytes, and one byte permute per 4 elements looks up
// their magnitudes in the scale's two table dwords; the sign bits are ORed in.
// Loads are streaming (each weight byte is read once); each lane writes 16
// contiguous bytes, so a wave's store covers 1 KiB.
#include "tis_common.h"
#include "tis_internal.h"

namespace tis {

// E4M3 byte of num * 2^t (num 1 or 3, t any exponent), rounded to nearest with
// ties to even, saturated at 448: the one place the format's rules live.
__device__ __forceinline__ uint32_t e4m3_of(int num, int t) {
  if (num == 1) {
    if (t > 8) return 0x7Eu;                         // beyond 448: saturate
    if (t >= -6) return (uint32_t)(t + 7) << 3;      // normal 1.000 * 2^t
    if (t >= -9) return 1u << (t + 9);               // subnormal: 1, 2 or 4 * 2^-9
    return 0u;                                       // 2^-10 is a tie: to 0 (even)
  }
  const int u = t + 1;                               // 3 * 2^t = 1.5 * 2^u
  if (u > 8) return 0x7Eu;
  if (u >= -6) return ((uint32_t)(u + 7) << 3) | 4u;  // normal 1.100 * 2^u
  if (t >= -9) return 3u << (t + 9);                 // 3 or 6 * 2^-9
  if (t == -10) return 2u;                           // 1.5 * 2^-9: a tie, to 2 (even)
  if (t == -11) return 1u;                           // 0.75 * 2^-9
  return 0u;
}

// E4M3 bytes of the 8 E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 at scale byte
// x: magnitudes 0-3 in the low dword, 4-7 in the high one.
__device__ __forceinline__ u32x2 magnitude_table(int x, int exp_offset) {
  if (x == 255) return u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
  const int s = x - 127 + exp_offset;
  // magnitude m = num * 2^e: 0.5 = 1*2^-1, 1 = 1*2^0, 1.5 = 3*2^-1, 2 = 1*2^1,
  // 3 = 3*2^0, 4 = 1*2^2, 6 = 3*2^1
  const uint32_t lo = (e4m3_of(1, s - 1) << 8) | (e4m3_of(1, s) << 16) | (e4m3_of(3, s - 1) << 24);
  const uint32_t hi = e4m3_of(1, s + 1) | (e4m3_of(3, s) << 8) | (e4m3_of(1, s + 2) << 16) |
                      (e4m3_of(3, s + 1) << 24);
  return u32x2{lo, hi};
}

// 8 elements (the nibbles of w, element 0 lowest) -> 8 E4M3 bytes (element 0
// in the lowest byte of the first dword).
__device__ __forceinline__ u32x2 convert8(uint32_t w, u32x2 tab) {
  u32x2 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t v = h ? w >> 16 : w;
    // nibbles n0 n1 n2 n3 of the low half-word into bytes 0..3: bytes of
    // a = v & 0x0f0f are (n0, n2), of b = (v >> 4) & 0x0f0f are (n1, n3)
    const uint32_t a = v & 0x0F0Fu, b = (v >> 4) & 0x0F0Fu;
    const uint32_t c = __builtin_amdgcn_perm(b, a, 0x05010400u);
    // magnitudes select bytes 0-3 (low table dword) or 4-7 (high dword)
    const uint32_t mag = __builtin_amdgcn_perm(tab.y, tab.x, c & 0x07070707u);
    const uint32_t sgn = (c & 0x08080808u) << 4;
    r[h] = mag | sgn;
  }
  return r;
}

constexpr int kConvThreads = 256;
constexpr int kConvSteps = 4;      // 16-element steps per thread and block
constexpr int64_t kConvBlockElems = (int64_t)kConvThreads * 16 * kConvSteps;

__global__ __launch_bounds__(kConvThreads) void mxfp4_to_fp8_kernel(Mxfp4Args a) {
  __shared__ u32x2 s_tab[256];
  const int tid = threadIdx.x;
  const int slot = blockIdx.y;
  const int id = a.expert_ids[slot];  // the same for the whole block
  if (id < 0 || id >= a.num_experts) return;
  const int64_t n = a.rows * a.cols;  // elements of one expert (a multiple of 32)
  const int64_t e_blk = (int64_t)blockIdx.x * kConvBlockElems;
  const uint8_t* pk = a.packed + (int64_t)id * (n / 2);
  const uint8_t* sc = a.scales + (int64_t)id * (n / 32);
  uint8_t* out = a.out + (int64_t)slot * n;

  // this thread's packed bytes and scales first, all in flight together
  u32x2 w[kConvSteps];
  uint32_t x[kConvSteps];
#pragma unroll
  for (int u = 0; u < kConvSteps; ++u) {
    int64_t e0 = e_blk + ((int64_t)u * kConvThreads + tid) * 16;
    if (e0 >= n) e0 = n - 16;  // re-read the last step (not stored)
    w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pk + e0 / 2));
    x[u] = __builtin_nontemporal_load(sc + e0 / 32);
  }
  s_tab[tid] = magnitude_table(tid, a.exp_offset);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kConvSteps; ++u) {
    const int64_t e0 = e_blk + ((int64_t)u * kConvThreads + tid) * 16;
    if (e0 >= n) break;
    const u32x2 tab = s_tab[x[u]];
    const u32x2 r0 = convert8(w[u].x, tab), r1 = convert8(w[u].y, tab);
    *reinterpret_cast<u32x4*>(out + e0) = u32x4{r0.x, r0.y, r1.x, r1.y};
  }
}

hipError_t launch_mxfp4_to_fp8(const Mxfp4Args& a, hipStream_t s) {
  const int64_t n = a.rows * a.cols;
  const int64_t blocks = (n + kConvBlockElems - 1) / kConvBlockElems;
  if (blocks > INT32_MAX || a.n_sel > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mxfp4_to_fp8_kernel, dim3((unsigned)blocks, (unsigned)a.n_sel),
                     dim3(kConvThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tis
