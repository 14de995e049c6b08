// Log-sum-exp merge of split partials -- flash decoding (Megatron-LM pull
// request 7211, commit "Replace the CuTe decode kernels with two Triton
// kernels": the slices of the top-k slots are merged).
//
//   M = max_s lse_s,  W = sum_s exp(lse_s - M),
//   out = sum_s exp(lse_s - M) o_s / W,  out_lse = M + ln W
//
// One wave per (row, head); lanes stride over the head dim, so each split's
// partial row is one coalesced read. bf16 output rounds to nearest even.

#include "dsa_kernels.h"

namespace dsa {

constexpr int kMergeWaves = 4;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int items, int d, int S,
    void* __restrict__ out, float* __restrict__ out_lse, int out_bf16) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (item >= items) return;
  const float* lse = part_lse + (size_t)item * S;
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, lse[s]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const bool any = M != -INFINITY;
  float W = 0.0f;
  if (any)
    for (int s = lane; s < S; s += 64) W += __expf(lse[s] - M);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) W += __shfl_xor(W, o);
  const float invW = any ? 1.0f / W : 0.0f;
  const float* po = part_o + (size_t)item * S * d;
  for (int e = lane; e < d; e += 64) {
    float acc = 0.0f;
    if (any)
      for (int s = 0; s < S; ++s) {
        const float ls = lse[s];
        if (ls != -INFINITY) acc = fmaf(__expf(ls - M), po[(size_t)s * d + e], acc);
      }
    const float v = acc * invW;
    if (out_bf16) static_cast<uint16_t*>(out)[(size_t)item * d + e] = f32_to_bf16_rne(v);
    else static_cast<float*>(out)[(size_t)item * d + e] = v;
  }
  if (out_lse && lane == 0) out_lse[item] = any ? M + __logf(W) : -INFINITY;
}

hipError_t launch_merge(const float* part_o, const float* part_lse, int rows, int hq, int d,
                        int num_splits, void* out, float* out_lse, bool out_bf16,
                        hipStream_t stream) {
  const int items = rows * hq;
  const int grid = (items + kMergeWaves - 1) / kMergeWaves;
  hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(64 * kMergeWaves), 0, stream, part_o,
                     part_lse, items, d, num_splits, out, out_lse, out_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dsa
