// Log-sum-exp merge of split partials -- flash decoding (Megatron-LM pull
// request 7211, commit "Replace the CuTe decode kernels with two Triton
// kernels": the slices of the top-k slots are merged).
//
//   M = max_s lse_s,  W = sum_s exp(lse_s - M),
//   out = sum_s exp(lse_s - M) o_s / W,  out_lse = M + ln W
//
// Up to kSeqSplits splits: one wave per (row, head), splits taken in order
// (the same operations, in the same order, as the merge inside the fused
// attention kernel, so the two agree bit for bit). The split log-sum-exps are
// read at wave-uniform addresses (scalar loads); each lane owns up to 4
// consecutive dims and issues the loads of up to 8 splits before using them.
// More splits (small batches split the slots widely): the four waves of a
// workgroup take every fourth split of one (row, head) and their partial
// merges are combined through LDS. bf16 output rounds to nearest even.

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

constexpr int kSeqSplits = 8;

// Partial merge of splits s0, s0 + step, ... < S of one (row, head): running
// max M, weight sum W and weighted sum acc against reference Mr.
template <int DPL>
__device__ __forceinline__ void merge_splits(const float* __restrict__ po,
                                             const float* __restrict__ lse, int S, int s0,
                                             int step, int d, int e0, bool mine, float Mr,
                                             float (&acc)[DPL], float& W) {
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
  W = 0.0f;
  for (int sb = s0; sb < S; sb += kMergeUnroll * step) {
    float v[kMergeUnroll][DPL];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = sb + u * step;
#pragma unroll
      for (int i = 0; i < DPL; ++i)
        v[u][i] = (s < S && mine && e0 + i < d) ? po[(size_t)s * d + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = sb + u * step;
      const float wgt = s < S ? __expf(lse[s] - Mr) : 0.0f;
      W += wgt;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(wgt, v[u][i], acc[i]);
    }
  }
}

template <int DPL>
__device__ __forceinline__ void merge_store(int item, int d, int e0, bool mine, bool any, float M,
                                            float W, const float (&acc)[DPL], void* out,
                                            float* out_lse, int out_bf16) {
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
  if (out_lse && (threadIdx.x & 63) == 0) out_lse[item] = any ? M + __logf(W) : -INFINITY;
}

// DPL: dims per lane (d <= 64 * DPL). One wave per (row, head), splits in order.
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
  float acc[DPL], W;
  merge_splits<DPL>(part_o + (size_t)item * S * d + e0, lse, S, 0, 1, d, e0, mine, Mr, acc, W);
  merge_store<DPL>(item, d, e0, mine, any, M, W, acc, out, out_lse, out_bf16);
}

// One workgroup per (row, head): wave w merges splits w, w + 4, ... against
// its own maximum, and wave 0 rescales and sums the four partial merges.
template <int DPL>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_wide_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int items, int d, int S,
    void* __restrict__ out, float* __restrict__ out_lse, int out_bf16) {
  __shared__ float acc_lds[kMergeWaves][64 * DPL];
  __shared__ float mw_lds[kMergeWaves][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x;
  const float* lse = part_lse + (size_t)item * S;
  float Mw = -INFINITY;
  for (int s = wave; s < S; s += kMergeWaves) Mw = fmaxf(Mw, lse[s]);
  const float Mr = Mw != -INFINITY ? Mw : 0.0f;
  const int e0 = lane * DPL;
  const bool mine = e0 < d;
  float acc[DPL], W;
  merge_splits<DPL>(part_o + (size_t)item * S * d + e0, lse, S, wave, kMergeWaves, d, e0, mine, Mr,
                    acc, W);
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc_lds[wave][lane * DPL + i] = acc[i];
  if (lane == 0) {
    mw_lds[wave][0] = Mw;
    mw_lds[wave][1] = W;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, mw_lds[w][0]);
  const bool any = M != -INFINITY;
  float tot[DPL], Wt = 0.0f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) tot[i] = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const float mw = mw_lds[w][0];
    const float f = (any && mw != -INFINITY) ? __expf(mw - M) : 0.0f;
    Wt = fmaf(f, mw_lds[w][1], Wt);
#pragma unroll
    for (int i = 0; i < DPL; ++i) tot[i] = fmaf(f, acc_lds[w][lane * DPL + i], tot[i]);
  }
  merge_store<DPL>(item, d, e0, mine, any, M, Wt, tot, out, out_lse, out_bf16);
}

hipError_t launch_merge(const float* part_o, const float* part_lse, int rows, int hq, int d,
                        int num_splits, void* out, float* out_lse, bool out_bf16,
                        hipStream_t stream) {
  const int items = rows * hq;
  const int bf = out_bf16 ? 1 : 0;
  const dim3 block(64 * kMergeWaves);
  if (num_splits > kSeqSplits) {
#define DSA_MERGE_WIDE(DPL_)                                                                  \
  hipLaunchKernelGGL(merge_wide_kernel<DPL_>, dim3(items), block, 0, stream, part_o, part_lse, \
                     items, d, num_splits, out, out_lse, bf)
    if (d <= 64) DSA_MERGE_WIDE(1);
    else if (d <= 128) DSA_MERGE_WIDE(2);
    else DSA_MERGE_WIDE(4);
#undef DSA_MERGE_WIDE
    return hipGetLastError();
  }
  const int grid = (items + kMergeWaves - 1) / kMergeWaves;
#define DSA_MERGE(DPL_)                                                                 \
  hipLaunchKernelGGL(merge_kernel<DPL_>, dim3(grid), block, 0, stream, part_o, part_lse, \
                     items, d, num_splits, out, out_lse, bf)
  if (d <= 64) DSA_MERGE(1);
  else if (d <= 128) DSA_MERGE(2);
  else DSA_MERGE(4);
#undef DSA_MERGE
  return hipGetLastError();
}

}  // namespace dsa
