// Building blocks of the radix-select top-k kernels: order-preserving keys
// of fp32 scores, wave and workgroup scans on DPP row operations, and the
// digit width of a radix pass. Shared by the one-pass / two-stage selection
// (topk.hip) and the histogram-driven selection (topk_hist.hip).
#pragma once

#include <type_traits>

#include "dsa_kernels.h"

namespace dsa {

constexpr int kTopkThreads = 1024;  // threads of the launched configuration
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popcount(uint32_t m) { return __popc(m); }
__device__ __forceinline__ int popcount(uint64_t m) { return __popcll(m); }
__device__ __forceinline__ int lowest_bit(uint32_t m) { return __ffs(m) - 1; }
__device__ __forceinline__ int lowest_bit(uint64_t m) { return __ffsll((unsigned long long)m) - 1; }

__device__ __forceinline__ uint32_t high_bits(uint32_t key, int shift) {
  return shift >= 32 ? 0u : (key >> shift);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Max and min over the wave, wave-uniform: butterflies inside each 16-lane
// row (quad permutes, half-row and row mirrors), then the four row results.
__device__ __forceinline__ void wave_max_min(uint32_t& mx, uint32_t& mn) {
  mx = max(mx, dpp_u32<0xB1>(mx));  // quad_perm [1,0,3,2]
  mn = min(mn, dpp_u32<0xB1>(mn));
  mx = max(mx, dpp_u32<0x4E>(mx));  // quad_perm [2,3,0,1]
  mn = min(mn, dpp_u32<0x4E>(mn));
  mx = max(mx, dpp_u32<0x141>(mx));  // row_half_mirror
  mn = min(mn, dpp_u32<0x141>(mn));
  mx = max(mx, dpp_u32<0x140>(mx));  // row_mirror
  mn = min(mn, dpp_u32<0x140>(mn));
  mx = max(max(lane_u32(mx, 0), lane_u32(mx, 16)), max(lane_u32(mx, 32), lane_u32(mx, 48)));
  mn = min(min(lane_u32(mn, 0), lane_u32(mn, 16)), min(lane_u32(mn, 32), lane_u32(mn, 48)));
}

// Bitwise OR and AND over the wave, wave-uniform (the same butterflies).
__device__ __forceinline__ void wave_or_and(uint32_t& o, uint32_t& a) {
  o |= dpp_u32<0xB1>(o);
  a &= dpp_u32<0xB1>(a);
  o |= dpp_u32<0x4E>(o);
  a &= dpp_u32<0x4E>(a);
  o |= dpp_u32<0x141>(o);
  a &= dpp_u32<0x141>(a);
  o |= dpp_u32<0x140>(o);
  a &= dpp_u32<0x140>(a);
  o = lane_u32(o, 0) | lane_u32(o, 16) | lane_u32(o, 32) | lane_u32(o, 48);
  a = lane_u32(a, 0) & lane_u32(a, 16) & lane_u32(a, 32) & lane_u32(a, 48);
}

// Inclusive prefix sum over the wave in lane order: shifts by 1, 2, 4, 8
// inside each 16-lane row (lanes shifted in from outside the row read 0),
// then the totals of the rows below.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_u32<0x111>(x);  // row_shr:1
  x += dpp_u32<0x112>(x);  // row_shr:2
  x += dpp_u32<0x114>(x);  // row_shr:4
  x += dpp_u32<0x118>(x);  // row_shr:8
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t r0 = lane_u32(x, 15), r1 = lane_u32(x, 31), r2 = lane_u32(x, 47);
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Exclusive prefix sum over the block in thread order; *total gets the sum.
// `sh` holds one word per wave; the caller gives each scan a slot that no
// other scan touches until a later barrier, so no barrier is needed after it.
template <int kTopkWaves>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const uint32_t x = sh[i];
    base += (i < wave) ? x : 0u;
    tot += x;
  }
  *total = tot;
  return base + incl - v;
}

// Exclusive prefix sums of two counts over the block in thread order, each
// at full 32-bit width (a chunk can hold 65536 keys that all tie, so the two
// counts cannot share one word); *ta / *tb get the totals. `sh` holds two
// words per wave, used as in block_exclusive_scan.
template <int kTopkWaves>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t* sh,
                                                      uint32_t* ea, uint32_t* eb, uint32_t* ta,
                                                      uint32_t* tb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_inclusive_scan(a);
  const uint32_t ib = wave_inclusive_scan(b);
  if (lane == 63) {
    sh[wave] = ia;
    sh[kTopkWaves + wave] = ib;
  }
  __syncthreads();
  uint32_t ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const uint32_t x = sh[i], y = sh[kTopkWaves + i];
    ba += (i < wave) ? x : 0u;
    bb += (i < wave) ? y : 0u;
    sa += x;
    sb += y;
  }
  *ea = ba + ia - a;
  *eb = bb + ib - b;
  *ta = sa;
  *tb = sb;
}

// Bins of a score histogram over the top 12 bits of the order key (sign,
// exponent and the top three mantissa bits); bin = order_key(score) >> 20.
constexpr int kHistBins = 1 << kDigitBits;
constexpr int kHistShift = 32 - kDigitBits;

}  // namespace dsa
