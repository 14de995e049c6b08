// GQA sparse attention over split k-slot slices (Megatron-LM pull request
// 7211, commit "Replace the CuTe decode kernels with two Triton kernels": one
// program handles all query heads of a KV group, reading each selected key and
// value once, and the top-k slots are split across programs; commit "Restore
// the upstream Blackwell FP32 probability reduction": probabilities stay fp32
// through the value reduction).
//
// One wave per (row, split, KV group). The split's slots are walked in tiles
// of 64:
//   * scores: lane j owns slot j of the tile. It reads the slot's position,
//     translates it through the block table, loads that key's row for the
//     group (d elements, contiguous), and dots it with each of the group's G
//     query heads (queries in LDS, read as broadcasts). bf16 keys use
//     v_dot2_f32_bf16: the bf16 products are exact and accumulate in fp32.
//   * online softmax per head in base 2 (the scale folds in log2 e), with one
//     wave max and one wave sum per head and tile; probabilities go to LDS.
//   * values: lane owns d/64 consecutive dims of the output; the tile's value
//     rows are loaded 16 at a time (each a coalesced d-element row read by the
//     whole wave) and accumulated with fp32 FMAs against the fp32
//     probabilities.
// Padding slots (-1) sit at the end of a row's selection; a tile with no
// valid slot ends the walk, and an empty split writes o = 0, lse = -inf.

#include "dsa_kernels.h"

namespace dsa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Element traits: Word is what one lane loads for its DPL output dims.
template <typename T, int DPL> struct Elem;
template <> struct Elem<uint16_t, 2> {
  typedef uint32_t Word;
  __device__ static float get(Word w, int i) { return i == 0 ? bf16_lo(w) : bf16_hi(w); }
};
template <> struct Elem<uint16_t, 1> {
  typedef uint16_t Word;
  __device__ static float get(Word w, int) { return __uint_as_float((uint32_t)w << 16); }
};
template <> struct Elem<float, 2> {
  typedef float2 Word;
  __device__ static float get(Word w, int i) { return i == 0 ? w.x : w.y; }
};
template <> struct Elem<float, 1> {
  typedef float Word;
  __device__ static float get(Word w, int) { return w; }
};

template <typename T, int D, int G>
__global__ __launch_bounds__(64) void sparse_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ idx, int hkv, int k, int page_shift, int max_pages,
    float scale_log2, int S, int chunk, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int DPL = D / 64;  // output dims per lane
  typedef Elem<T, DPL> E;
  typedef typename E::Word Word;
  constexpr int QW = kBf16 ? D / 2 : D;  // 32-bit words per query head row
  __shared__ __attribute__((aligned(16))) uint32_t q_lds[G * QW];
  __shared__ float p_lds[64 * G];
  __shared__ uint32_t row_lds[64];

  const int lane = threadIdx.x;
  const int g = blockIdx.x % hkv;
  const int rs = blockIdx.x / hkv;
  const int s = rs % S;
  const int r = rs / S;
  const int hq = hkv * G;
  const int a = min(k, s * chunk);
  const int b = min(k, a + chunk);
  const int page_mask = (1 << page_shift) - 1;

  {
    const uint32_t* qsrc =
        reinterpret_cast<const uint32_t*>(q + ((size_t)r * hq + (size_t)g * G) * D);
    for (int i = lane; i < G * QW; i += 64) q_lds[i] = qsrc[i];
  }
  __syncthreads();

  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.0f;
  }

  const int32_t* btr = bt + (size_t)row_req[r] * max_pages;
  const int32_t* ir = idx + (size_t)r * k;
  const size_t kv_stride = (size_t)hkv * D;

  for (int t0 = a; t0 < b; t0 += 64) {
    const int slot = t0 + lane;
    const int pos = slot < b ? ir[slot] : -1;
    const bool valid = pos >= 0;
    if (__ballot(valid) == 0) break;
    uint32_t krow = 0xFFFFFFFFu;
    if (valid) krow = ((uint32_t)btr[pos >> page_shift] << page_shift) | (uint32_t)(pos & page_mask);

    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.0f;
    if (valid) {
      const uint4* kp = reinterpret_cast<const uint4*>(kc + (size_t)krow * kv_stride + (size_t)g * D);
      constexpr int NV = QW / 4;  // uint4 per key row
      uint4 kv[NV];
#pragma unroll
      for (int c = 0; c < NV; ++c) kv[c] = kp[c];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4* qh = reinterpret_cast<const uint4*>(q_lds + h * QW);
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          const uint4 qv = qh[c];
          if constexpr (kBf16) {
            acc = dot2_bf16(kv[c].x, qv.x, acc);
            acc = dot2_bf16(kv[c].y, qv.y, acc);
            acc = dot2_bf16(kv[c].z, qv.z, acc);
            acc = dot2_bf16(kv[c].w, qv.w, acc);
          } else {
            acc = fmaf(__uint_as_float(kv[c].x), __uint_as_float(qv.x), acc);
            acc = fmaf(__uint_as_float(kv[c].y), __uint_as_float(qv.y), acc);
            acc = fmaf(__uint_as_float(kv[c].z), __uint_as_float(qv.z), acc);
            acc = fmaf(__uint_as_float(kv[c].w), __uint_as_float(qv.w), acc);
          }
        }
        sc[h] = acc * scale_log2;
      }
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = wave_max_f32(valid ? sc[h] : -INFINITY);
      const float mn = fmaxf(m[h], mt);
      const float alpha = (m[h] == -INFINITY) ? 0.0f : exp2f(m[h] - mn);
      const float p = valid ? exp2f(sc[h] - mn) : 0.0f;
      l[h] = l[h] * alpha + wave_sum_f32(p);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] *= alpha;
      m[h] = mn;
      p_lds[lane * G + h] = p;
    }
    row_lds[lane] = krow;
    __syncthreads();

    const T* vbase = vc + (size_t)g * D + (size_t)lane * DPL;
#pragma unroll 1
    for (int j0 = 0; j0 < 64; j0 += 16) {
      Word vw[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const uint32_t rj = row_lds[j0 + jj];
        if (rj != 0xFFFFFFFFu) vw[jj] = *reinterpret_cast<const Word*>(vbase + (size_t)rj * kv_stride);
        else vw[jj] = Word{};
      }
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = p_lds[(j0 + jj) * G + h];
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[h][e] = fmaf(p, E::get(vw[jj], e), o[h][e]);
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t head = (size_t)r * hq + (size_t)g * G + h;
    const bool any = l[h] > 0.0f;
    const float inv = any ? 1.0f / l[h] : 0.0f;
    float* po = part_o + (head * S + s) * D + (size_t)lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) po[e] = o[h][e] * inv;
    if (lane == 0) part_lse[head * S + s] = any ? (m[h] + __log2f(l[h])) * kLn2 : -INFINITY;
  }
}

template <typename T>
static hipError_t launch_attn_t(const T* q, const T* kc, const T* vc, const int32_t* bt,
                                const int32_t* row_req, const int32_t* idx, int rows, int hq,
                                int hkv, int d, int k, int page_shift, int max_pages, float scale,
                                int S, float* part_o, float* part_lse, hipStream_t stream) {
  const int G = hq / hkv;
  const int chunk = (k + S - 1) / S;
  const dim3 grid((unsigned)rows * S * hkv);
  const float sl2 = scale * kLog2e;
#define DSA_ATTN(D_, G_)                                                                     \
  hipLaunchKernelGGL((sparse_attn_kernel<T, D_, G_>), grid, dim3(64), 0, stream, q, kc, vc, bt, \
                     row_req, idx, hkv, k, page_shift, max_pages, sl2, S, chunk, part_o,      \
                     part_lse)
#define DSA_ATTN_G(D_)                  \
  switch (G) {                          \
    case 1: DSA_ATTN(D_, 1); break;     \
    case 2: DSA_ATTN(D_, 2); break;     \
    case 4: DSA_ATTN(D_, 4); break;     \
    case 8: DSA_ATTN(D_, 8); break;     \
    case 16: DSA_ATTN(D_, 16); break;   \
    default: return hipErrorInvalidValue; \
  }
  if (d == 128) {
    DSA_ATTN_G(128);
  } else if (d == 64) {
    DSA_ATTN_G(64);
  } else {
    return hipErrorInvalidValue;
  }
#undef DSA_ATTN_G
#undef DSA_ATTN
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* bt,
                              const int32_t* row_req, const int32_t* idx, int rows, int hq,
                              int hkv, int d, int k, int page_shift, int max_pages, float scale,
                              int num_splits, float* part_o, float* part_lse, bool bf16,
                              hipStream_t stream) {
  if (bf16)
    return launch_attn_t(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                         static_cast<const uint16_t*>(vc), bt, row_req, idx, rows, hq, hkv, d, k,
                         page_shift, max_pages, scale, num_splits, part_o, part_lse, stream);
  return launch_attn_t(static_cast<const float*>(q), static_cast<const float*>(kc),
                       static_cast<const float*>(vc), bt, row_req, idx, rows, hq, hkv, d, k,
                       page_shift, max_pages, scale, num_splits, part_o, part_lse, stream);
}

}  // namespace dsa
