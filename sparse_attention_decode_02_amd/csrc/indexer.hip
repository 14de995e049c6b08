// Lightning-indexer scores over paged key tiles (Megatron-LM pull request
// 7211, commit "Replace the CuTe decode kernels with two Triton kernels":
// indexer scores stream page-contiguous key tiles on the matrix cores, and a
// request's programs stride over its row only up to its length):
//
//   scores[r][s] = sum_h w[r][h] * max(0, qI[r][h] . kI[req(r)][s]),  s < L_r
//
// bf16 path (MFMA): per row the contraction is (heads x dim) . (dim x keys).
// One wave computes a 32-key tile for all heads with
// v_mfma_f32_32x32x16_bf16, heads on the M side (32 per head tile) and keys
// on the N side. A lane owns one key (lane % 32) and one half of its dims
// (lane / 32), so its B fragments are 64 contiguous bytes per MFMA step of
// that key's row: the k index of MFMA step kk, lane half hf, element e is
// dim hf * D/2 + kk * 8 + e, for both operands. After the MFMAs a lane holds
// 16 heads of its key per head tile; ReLU, the head weight and the head sum
// run in fp32 registers and one cross-half exchange finishes the key.
// Products of bf16 are exact and the configs' dyadic integers accumulate
// exactly in fp32, in any order.
//
// fp32 path (VALU): one thread per key, fp32 FMA, queries in LDS.
//
// Work: a workgroup takes (score block, key chunk); the rows of a block
// belong to one request and are scored one after another against the same
// chunk, so the chunk's keys are re-read from cache, not HBM. Chunks past a
// row's length exit at once, so the launch depends only on (blocks, width)
// while the work follows the real lengths.

#include "dsa_kernels.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kIdxThreads = 256;  // 4 waves
constexpr int kTileKeys = 32;     // keys per MFMA tile (N of 32x32x16)

template <int HT, int DI>
__global__ __launch_bounds__(kIdxThreads, 2) void indexer_mfma_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w,
    const uint16_t* __restrict__ kc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ row_req, const int32_t* __restrict__ row_len,
    const int32_t* __restrict__ blocks, float* __restrict__ scores, int width, int page_shift,
    int max_pages, int chunk_keys, int chunks, int total) {
  constexpr int H = HT * 32;
  constexpr int KS = DI / 16;  // MFMA steps per head tile
  constexpr int HALF = DI / 2;
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[H * DI];
  __shared__ float w_lds[H];

  const int item = xcd_contiguous(blockIdx.x, total);
  const int b = item / chunks;
  const int chunk0 = (item - b * chunks) * chunk_keys;
  int first = b, nrows = 1;
  if (blocks) {
    first = blocks[2 * b];
    nrows = blocks[2 * b + 1];
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kl = lane & 31, hf = lane >> 5;
  const int page_mask = (1 << page_shift) - 1;

  for (int rr = 0; rr < nrows; ++rr) {
    const int r = first + rr;
    const int L = row_len[r];
    if (chunk0 >= L) continue;  // uniform over the workgroup
    const int req = row_req[r];
    __syncthreads();
    {
      const uint4* src = reinterpret_cast<const uint4*>(qI + (size_t)r * H * DI);
      uint4* dst = reinterpret_cast<uint4*>(q_lds);
      for (int i = tid; i < H * DI / 8; i += kIdxThreads) dst[i] = src[i];
      for (int i = tid; i < H; i += kIdxThreads) w_lds[i] = w[(size_t)r * H + i];
    }
    __syncthreads();

    bf16x8 qf[HT][KS];
    float wr[HT][16];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        qf[t][kk] = *reinterpret_cast<const bf16x8*>(&q_lds[(t * 32 + kl) * DI + hf * HALF + kk * 8]);
#pragma unroll
      for (int j = 0; j < 16; ++j) wr[t][j] = w_lds[t * 32 + (j >> 2) * 8 + hf * 4 + (j & 3)];
    }

    const int32_t* btr = bt + (size_t)req * max_pages;
    const int end = min(L, chunk0 + chunk_keys);
    float* out = scores + (size_t)r * width;
    for (int base = chunk0 + wave * kTileKeys; base < end; base += 4 * kTileKeys) {
      const int s = base + kl;
      bf16x8 kf[KS];
      if (s < L) {
        const int page = btr[s >> page_shift];
        const size_t krow = ((size_t)page << page_shift) | (size_t)(s & page_mask);
        const bf16x8* p = reinterpret_cast<const bf16x8*>(kc + krow * DI + hf * HALF);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) kf[kk] = p[kk];
      } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) kf[kk] = bf16x8{};
      }
      float part = 0.0f;
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][kk], kf[kk], acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 16; ++j) part += wr[t][j] * fmaxf(acc[j], 0.0f);
      }
      part += __shfl_xor(part, 32);
      if (hf == 0 && s < L) out[s] = part + 0.0f;
    }
  }
}

template <int DI>
__global__ __launch_bounds__(kIdxThreads) void indexer_f32_kernel(
    const float* __restrict__ qI, const float* __restrict__ w, const float* __restrict__ kc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ blocks,
    float* __restrict__ scores, int width, int H, int page_shift, int max_pages, int chunk_keys,
    int chunks, int total) {
  __shared__ float q_lds[64 * DI];
  __shared__ float w_lds[64];
  const int item = xcd_contiguous(blockIdx.x, total);
  const int b = item / chunks;
  const int chunk0 = (item - b * chunks) * chunk_keys;
  int first = b, nrows = 1;
  if (blocks) {
    first = blocks[2 * b];
    nrows = blocks[2 * b + 1];
  }
  const int tid = threadIdx.x;
  const int page_mask = (1 << page_shift) - 1;
  for (int rr = 0; rr < nrows; ++rr) {
    const int r = first + rr;
    const int L = row_len[r];
    if (chunk0 >= L) continue;
    const int req = row_req[r];
    __syncthreads();
    for (int i = tid; i < H * DI; i += kIdxThreads) q_lds[i] = qI[(size_t)r * H * DI + i];
    for (int i = tid; i < H; i += kIdxThreads) w_lds[i] = w[(size_t)r * H + i];
    __syncthreads();
    const int end = min(L, chunk0 + chunk_keys);
    for (int s = chunk0 + tid; s < end; s += kIdxThreads) {
      const int page = bt[(size_t)req * max_pages + (s >> page_shift)];
      const float* kp = kc + (((size_t)page << page_shift) | (size_t)(s & page_mask)) * DI;
      float kv[DI];
#pragma unroll
      for (int j = 0; j < DI; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(kp + j);
        kv[j] = v.x;
        kv[j + 1] = v.y;
        kv[j + 2] = v.z;
        kv[j + 3] = v.w;
      }
      float tot = 0.0f;
      for (int h = 0; h < H; ++h) {
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < DI; ++j) dot = fmaf(q_lds[h * DI + j], kv[j], dot);
        tot += w_lds[h] * fmaxf(dot, 0.0f);
      }
      scores[(size_t)r * width + s] = tot + 0.0f;
    }
  }
}

int indexer_chunk_keys(int num_blocks, int width) {
  // Enough workgroups to cover 256 CUs several times over, with chunks that
  // still amortize the per-row query load.
  int chunk = 1024;
  while (chunk > 128 && (long long)num_blocks * ((width + chunk - 1) / chunk) < 2048) chunk >>= 1;
  return chunk;
}

hipError_t launch_indexer_bf16(const void* q_idx, const float* w, const void* kcache,
                               const int32_t* bt, const int32_t* row_req, const int32_t* row_len,
                               const int32_t* blocks, int num_blocks, float* scores, int width,
                               int num_heads, int head_dim, int page_shift, int max_pages,
                               hipStream_t stream) {
  const int chunk = indexer_chunk_keys(num_blocks, width);
  const int chunks = (width + chunk - 1) / chunk;
  const int total = num_blocks * chunks;
  const auto* q = static_cast<const uint16_t*>(q_idx);
  const auto* k = static_cast<const uint16_t*>(kcache);
#define DSA_IDX_LAUNCH(HT, DI)                                                                 \
  hipLaunchKernelGGL((indexer_mfma_kernel<HT, DI>), dim3(total), dim3(kIdxThreads), 0, stream, \
                     q, w, k, bt, row_req, row_len, blocks, scores, width, page_shift,         \
                     max_pages, chunk, chunks, total)
  if (num_heads == 64 && head_dim == 128) DSA_IDX_LAUNCH(2, 128);
  else if (num_heads == 32 && head_dim == 128) DSA_IDX_LAUNCH(1, 128);
  else if (num_heads == 64 && head_dim == 64) DSA_IDX_LAUNCH(2, 64);
  else if (num_heads == 32 && head_dim == 64) DSA_IDX_LAUNCH(1, 64);
  else return hipErrorInvalidValue;
#undef DSA_IDX_LAUNCH
  return hipGetLastError();
}

hipError_t launch_indexer_f32(const float* q_idx, const float* w, const float* kcache,
                              const int32_t* bt, const int32_t* row_req, const int32_t* row_len,
                              const int32_t* blocks, int num_blocks, float* scores, int width,
                              int num_heads, int head_dim, int page_shift, int max_pages,
                              hipStream_t stream) {
  const int chunk = 256;
  const int chunks = (width + chunk - 1) / chunk;
  const int total = num_blocks * chunks;
#define DSA_IDX_F32(DI)                                                                       \
  hipLaunchKernelGGL((indexer_f32_kernel<DI>), dim3(total), dim3(kIdxThreads), 0, stream, q_idx, \
                     w, kcache, bt, row_req, row_len, blocks, scores, width, num_heads,        \
                     page_shift, max_pages, chunk, chunks, total)
  if (head_dim == 32) DSA_IDX_F32(32);
  else if (head_dim == 64) DSA_IDX_F32(64);
  else if (head_dim == 128) DSA_IDX_F32(128);
  else return hipErrorInvalidValue;
#undef DSA_IDX_F32
  return hipGetLastError();
}

}  // namespace dsa
