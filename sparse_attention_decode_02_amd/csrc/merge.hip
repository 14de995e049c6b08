// Log-sum-exp merge of split partials -- flash decoding (Megatron-LM pull
// request 7211, commit "Replace the CuTe decode kernels with two Triton
// kernels": the slices of the top-k slots are merged).
//
//   M = max_s lse_s,  W = sum_s exp(lse_s - M),
//   out = sum_s exp(lse_s - M) o_s / W,  out_lse = M + ln W
//
// One wave per (row, head). The split log-sum-exps are read at wave-uniform
// addresses (scalar loads); each lane owns up to 4 consecutive dims and issues
// the loads of up to 8 splits before using them. bf16 output rounds to
// nearest even.

#include "dsa_kernels.h"

namespace dsa {

constexpr int kMergeWaves = 4;
constexpr int kMergeUnroll = 8;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// DPL: dims per lane (d <= 64 * DPL).
template <int DPL>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int items, int d, int S,
    void* __restrict__ out, float* __restrict__ out_lse, int out_bf16) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (item >= items) return;
  const float* lse = part_lse + (size_t)item * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lse[s]);
  const bool any = M != -INFINITY;
  const float Mr = any ? M : 0.0f;  // every weight is exp(-inf - 0) = 0 when nothing is valid
  const int e0 = lane * DPL;
  const bool mine = e0 < d;
  const float* po = part_o + (size_t)item * S * d + e0;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
  float W = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kMergeUnroll) {
    float v[kMergeUnroll][DPL];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = s0 + u;
#pragma unroll
      for (int i = 0; i < DPL; ++i)
        v[u][i] = (s < S && mine && e0 + i < d) ? po[(size_t)s * d + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = s0 + u;
      const float wgt = s < S ? __expf(lse[s] - Mr) : 0.0f;
      W += wgt;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(wgt, v[u][i], acc[i]);
    }
  }
  const float invW = any ? 1.0f / W : 0.0f;
  if (mine) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      if (e0 + i >= d) break;
      const float x = acc[i] * invW;
      if (out_bf16) static_cast<uint16_t*>(out)[(size_t)item * d + e0 + i] = f32_to_bf16_rne(x);
      else static_cast<float*>(out)[(size_t)item * d + e0 + i] = x;
    }
  }
  if (out_lse && lane == 0) out_lse[item] = any ? M + __logf(W) : -INFINITY;
}

hipError_t launch_merge(const float* part_o, const float* part_lse, int rows, int hq, int d,
                        int num_splits, void* out, float* out_lse, bool out_bf16,
                        hipStream_t stream) {
  const int items = rows * hq;
  const int grid = (items + kMergeWaves - 1) / kMergeWaves;
  const int bf = out_bf16 ? 1 : 0;
  if (d <= 64)
    hipLaunchKernelGGL(merge_kernel<1>, dim3(grid), dim3(64 * kMergeWaves), 0, stream, part_o,
                       part_lse, items, d, num_splits, out, out_lse, bf);
  else if (d <= 128)
    hipLaunchKernelGGL(merge_kernel<2>, dim3(grid), dim3(64 * kMergeWaves), 0, stream, part_o,
                       part_lse, items, d, num_splits, out, out_lse, bf);
  else
    hipLaunchKernelGGL(merge_kernel<4>, dim3(grid), dim3(64 * kMergeWaves), 0, stream, part_o,
                       part_lse, items, d, num_splits, out, out_lse, bf);
  return hipGetLastError();
}

}  // namespace dsa
