// Lightning-indexer scores over paged key tiles (Megatron-LM pull request
// 7211, commit "Replace the CuTe decode kernels with two Triton kernels":
// indexer scores stream page-contiguous key tiles on the matrix cores, and a
// request's programs stride over its row only up to its length):
//
//   scores[r][s] = sum_h w[r][h] * max(0, qI[r][h] . kI[req(r)][s]),  s < L_r
//
// bf16 path (MFMA): per row the contraction is (heads x dim) . (dim x keys).
// One wave computes a 16-key tile for all heads with v_mfma_f32_16x16x32_bf16
// (heads as rows, 16 per head tile; keys as columns). Four lanes share a key
// and read 64 contiguous bytes of its row per MFMA step; three key tiles
// rotate through registers so two are in flight while one is on the matrix
// cores. The query fragments are read from LDS for every tile rather than
// held in registers, which leaves room for four waves per SIMD. After the
// MFMAs a lane holds 4 consecutive heads of its key per head
// tile; ReLU, the head weight and the head sum run in fp32 registers and two
// row swaps (v_permlane16_swap, v_permlane32_swap) finish the key.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxThreads = 256;  // 4 waves
constexpr int kTileKeys = 16;     // keys per MFMA tile (N of 16x16x32)
constexpr int kKeyBufs = 3;       // key tiles per wave: 2 in flight + 1 on the matrix cores
constexpr int kMaxChunkKeys = 2048;  // keys per workgroup chunk, at most (scores staged in LDS)

// max(x, 0) as a signed-integer max of the bits: one VALU op, -0.0 -> +0.0.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// x summed over the four 16-lane rows of the wave (every lane gets the total).
__device__ __forceinline__ float sum_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// MFMA layout (v_mfma_f32_16x16x32_bf16): lane l feeds A row l%16 and B
// column l%16 with k = (l/16)*8 + e, e < 8, and gets D rows (l/16)*4 + i,
// i < 4, of column l%16. Heads are the rows (16 per head tile), keys the
// columns. The k index of step kk, lane group g = l/16, element e is dim
// kk*32 + g*8 + e for both operands, so the four lanes of a key read 64
// contiguous bytes of its row per step.
template <int HT, int DI>
__global__ __launch_bounds__(kIdxThreads, 4) void indexer_mfma_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w,
    const uint16_t* __restrict__ kc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ row_req, const int32_t* __restrict__ row_len,
    const int32_t* __restrict__ blocks, float* __restrict__ scores, int width, int page_shift,
    int max_pages, int chunk_keys, int chunks, int total, int score_row0) {
  constexpr int H = HT * 16;
  constexpr int KS = DI / 32;  // MFMA steps per head tile
  constexpr int QST = DI + 8;  // padded LDS row (elements): the 16 rows read together hit distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[H * QST];
  __shared__ __attribute__((aligned(16))) float w_lds[H];
  __shared__ __attribute__((aligned(16))) float s_lds[kMaxChunkKeys];  // the chunk's scores

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
  const int kl = lane & 15, grp = lane >> 4;
  const int page_mask = (1 << page_shift) - 1;

  // Wave-uniform pieces (readfirstlane makes them SGPRs, so the page lookups
  // below are scalar loads: they wait on the scalar counter and never on the
  // key loads still in flight).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  constexpr int kStep = 4 * kTileKeys;  // the workgroup's 4 waves interleave tiles
  constexpr int QV = H * DI / 8 / kIdxThreads;  // uint4 of the query block per thread
  static_assert(QV * kIdxThreads * 8 == H * DI, "query block must split evenly over the threads");

  for (int rr = 0; rr < nrows; ++rr) {
    const int r = first + rr;
    const int L = row_len[r];
    if (chunk0 >= L) continue;  // uniform over the workgroup
    const int req = row_req[r];
    const int32_t* btr = bt + (size_t)req * max_pages;
    const int end = min(L, chunk0 + chunk_keys);
    float* out = scores + (size_t)(r - score_row0) * width;  // rows of a window from its first

    // Key fragments of the 16-key tile at `base` (base is wave-uniform). The
    // tile lies inside one page (page size >= 16), whose number is one scalar
    // load. Loads are unconditional -- positions past the workgroup's chunk
    // re-read its last key (a cache hit) and are never stored -- so the load
    // counter stays exact and a prefetch is never waited on early.
    auto load_tile = [&](int base, bf16x8 (&kf)[KS]) {
      const int page = btr[min(base, end - 1) >> page_shift];
      const int s = min(base + kl, end - 1);
      const size_t krow = ((size_t)page << page_shift) | (size_t)(s & page_mask);
      const bf16x8* p = reinterpret_cast<const bf16x8*>(kc + krow * DI + grp * 8);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) kf[kk] = p[kk * 4];
    };

    // Prologue: the first key tiles, then the query block and head weights,
    // all in flight together; one wait covers them before the query goes to
    // LDS.
    const int base0 = chunk0 + wv * kTileKeys;
    const int ntiles = (end - base0 + kStep - 1) / kStep;  // this wave's tiles (may be <= 0)
    bf16x8 kbuf[kKeyBufs][KS];
#pragma unroll
    for (int i = 0; i < kKeyBufs - 1; ++i) load_tile(base0 + i * kStep, kbuf[i]);
    __syncthreads();  // the previous row's readers are done with q_lds / w_lds
    {
      const uint4* src = reinterpret_cast<const uint4*>(qI + (size_t)r * H * DI);
      uint4 qreg[QV];
#pragma unroll
      for (int i = 0; i < QV; ++i) qreg[i] = src[tid + i * kIdxThreads];
      const float wv_ = tid < H ? w[(size_t)r * H + tid] : 0.0f;
#pragma unroll
      for (int i = 0; i < QV; ++i) {
        const int e = tid + i * kIdxThreads;
        const int h = e / (DI / 8), c = e - h * (DI / 8);
        *reinterpret_cast<uint4*>(&q_lds[h * QST + c * 8]) = qreg[i];
      }
      if (tid < H) w_lds[tid] = wv_;
    }
    __syncthreads();

    float4 wr[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) wr[t] = *reinterpret_cast<const float4*>(&w_lds[t * 16 + grp * 4]);
    const int qoff0 = kl * QST + grp * 8;

    auto score_tile = [&](int base, const bf16x8 (&kf)[KS]) {
      // The empty asm makes the LDS offset opaque, so the compiler cannot hoist
      // the query reads out of the tile loop into registers.
      int qoff = qoff0;
      asm volatile("" : "+v"(qoff));
      float part = 0.0f;
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        f32x4 acc = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const bf16x8 qv = *reinterpret_cast<const bf16x8*>(&q_lds[t * 16 * QST + kk * 32 + qoff]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv, kf[kk], acc, 0, 0, 0);
        }
        part = fmaf(wr[t].x, relu(acc[0]), part);
        part = fmaf(wr[t].y, relu(acc[1]), part);
        part = fmaf(wr[t].z, relu(acc[2]), part);
        part = fmaf(wr[t].w, relu(acc[3]), part);
      }
      part = sum_rows(part);
      const int s = base + kl;
      if (grp == 0 && s < L) s_lds[s - chunk0] = part + 0.0f;
    };

    // kKeyBufs key-fragment buffers in rotation: while one tile runs on the
    // matrix cores the next two are in flight. The trip count is fixed and
    // every load unconditional, so each wait covers exactly the tile in use.
    for (int it = 0; it < ntiles; it += kKeyBufs) {
#pragma unroll
      for (int u = 0; u < kKeyBufs; ++u) {
        const int cur = base0 + (it + u) * kStep;
        load_tile(cur + (kKeyBufs - 1) * kStep, kbuf[(u + kKeyBufs - 1) % kKeyBufs]);
        if (it + u < ntiles) score_tile(cur, kbuf[u]);
      }
    }
    // The chunk's scores leave in whole lines with streaming stores once the
    // chunk is done: writing each tile's 16 scores as they come costs a few
    // percent of the kernel's time against the key reads.
    __syncthreads();
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int nk = end - chunk0;
    for (int i = tid * 4; i < nk; i += kIdxThreads * 4) {
      if (i + 4 <= nk) {
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4v*>(&s_lds[i]),
                                    reinterpret_cast<f32x4v*>(out + chunk0 + i));
      } else {
        for (int j = i; j < nk; ++j) out[chunk0 + j] = s_lds[j];
      }
    }
  }
}

template <int DI>
__global__ __launch_bounds__(kIdxThreads) void indexer_f32_kernel(
    const float* __restrict__ qI, const float* __restrict__ w, const float* __restrict__ kc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ blocks,
    float* __restrict__ scores, int width, int H, int page_shift, int max_pages, int chunk_keys,
    int chunks, int total, int score_row0) {
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
      scores[(size_t)(r - score_row0) * width + s] = tot + 0.0f;
    }
  }
}

int device_capacity(const void* kernel, int block) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return 0;
  return cus * per_cu;
}

static const void* indexer_kernel_ptr(int num_heads, int head_dim) {
  if (num_heads == 64 && head_dim == 128) return (const void*)indexer_mfma_kernel<4, 128>;
  if (num_heads == 32 && head_dim == 128) return (const void*)indexer_mfma_kernel<2, 128>;
  if (num_heads == 64 && head_dim == 64) return (const void*)indexer_mfma_kernel<4, 64>;
  if (num_heads == 32 && head_dim == 64) return (const void*)indexer_mfma_kernel<2, 64>;
  return nullptr;
}

int indexer_chunk_keys(int num_blocks, int width, int num_heads, int head_dim, bool full) {
  // About one round of workgroups over the device: a kernel whose grid is a
  // small multiple of what runs at once leaves most of the chip idle in its
  // last round. Chunks are capped so that long rows spread over many
  // workgroups: with fewer blocks than the device holds, ragged lengths leave
  // a few long rows as the tail, so the cap is 1024 keys -- unless the caller
  // knows the rows fill the score width (`full`), where 2048-key chunks have
  // no tail to balance and load the query block half as often; with more
  // blocks than the device holds, 2048.
  const void* kern = indexer_kernel_ptr(num_heads, head_dim);
  int cap = kern ? device_capacity(kern, kIdxThreads) : 0;
  if (cap <= 0) cap = 1024;
  const int per_block = max(1, cap / max(1, num_blocks));
  const int max_chunk = (per_block > 1 && !full) ? 1024 : kMaxChunkKeys;
  int chunk = (width + per_block - 1) / per_block;
  chunk = ((chunk + 63) / 64) * 64;
  // At least 256 keys (four tiles per wave) to amortize the query load.
  return max(256, min(max_chunk, chunk));
}

hipError_t launch_indexer_bf16(const void* q_idx, const float* w, const void* kcache,
                               const int32_t* bt, const int32_t* row_req, const int32_t* row_len,
                               const int32_t* blocks, int num_blocks, float* scores, int width,
                               int num_heads, int head_dim, int page_shift, int max_pages,
                               bool full, int score_row0, hipStream_t stream) {
  const int chunk = indexer_chunk_keys(num_blocks, width, num_heads, head_dim, full);
  const int chunks = (width + chunk - 1) / chunk;
  const int total = num_blocks * chunks;
  const auto* q = static_cast<const uint16_t*>(q_idx);
  const auto* k = static_cast<const uint16_t*>(kcache);
#define DSA_IDX_LAUNCH(HT, DI)                                                                 \
  hipLaunchKernelGGL((indexer_mfma_kernel<HT, DI>), dim3(total), dim3(kIdxThreads), 0, stream, \
                     q, w, k, bt, row_req, row_len, blocks, scores, width, page_shift,         \
                     max_pages, chunk, chunks, total, score_row0)
  if (num_heads == 64 && head_dim == 128) DSA_IDX_LAUNCH(4, 128);
  else if (num_heads == 32 && head_dim == 128) DSA_IDX_LAUNCH(2, 128);
  else if (num_heads == 64 && head_dim == 64) DSA_IDX_LAUNCH(4, 64);
  else if (num_heads == 32 && head_dim == 64) DSA_IDX_LAUNCH(2, 64);
  else return hipErrorInvalidValue;
#undef DSA_IDX_LAUNCH
  return hipGetLastError();
}

hipError_t launch_indexer_f32(const float* q_idx, const float* w, const float* kcache,
                              const int32_t* bt, const int32_t* row_req, const int32_t* row_len,
                              const int32_t* blocks, int num_blocks, float* scores, int width,
                              int num_heads, int head_dim, int page_shift, int max_pages,
                              int score_row0, hipStream_t stream) {
  const int chunk = 256;
  const int chunks = (width + chunk - 1) / chunk;
  const int total = num_blocks * chunks;
#define DSA_IDX_F32(DI)                                                                       \
  hipLaunchKernelGGL((indexer_f32_kernel<DI>), dim3(total), dim3(kIdxThreads), 0, stream, q_idx, \
                     w, kcache, bt, row_req, row_len, blocks, scores, width, num_heads,        \
                     page_shift, max_pages, chunk, chunks, total, score_row0)
  if (head_dim == 32) DSA_IDX_F32(32);
  else if (head_dim == 64) DSA_IDX_F32(64);
  else if (head_dim == 128) DSA_IDX_F32(128);
  else return hipErrorInvalidValue;
#undef DSA_IDX_F32
  return hipGetLastError();
}

}  // namespace dsa
