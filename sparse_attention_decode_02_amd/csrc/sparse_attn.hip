// GQA sparse attention over split k-slot slices (Megatron-LM pull request
// 7211, commit "Replace the CuTe decode kernels with two Triton kernels": one
// program handles all query heads of a KV group, reading each selected key and
// value once, and the top-k slots are split across programs; commit "Restore
// the upstream Blackwell FP32 probability reduction": probabilities stay fp32
// through the value reduction).
//
// One wave per (row, split, KV group); in the merged variant the splits of one
// (row, KV group) are the waves of one workgroup and are merged through LDS at
// the end (no partials in HBM, no second launch). bf16 rows with d = 128 and
// eight query heads per KV group (the decode shape of the method's models)
// run on the matrix cores (sparse_attn_mx_kernel below); every other shape
// runs on the vector kernel, whose waves walk the split's slots in tiles of
// 32 tokens, two lanes per token:
//   * addresses: a prologue translates up to 512 selected positions through
//     the block table into cache row ids in LDS (two dependent round trips
//     per span, not per tile); tiles past the span's last selected slot are
//     skipped.
//   * pipelining: V of tile t is requested before tile t's scores, K of tile
//     t+1 before tile t's value sums; every load is unconditional (padding
//     reads cache row 0 with probability 0), so each wait covers exactly the
//     data in use.
//   * K: lane t reads the first half of token t's row for the group, lane
//     t + 32 the second half (two 128-byte runs per 256-byte bf16 row).
//   * V: for each token j the whole wave reads its row (lane l gets dims
//     [l*d/64, (l+1)*d/64)), addressed from token j's row id taken from lane j
//     as a wave-uniform value, so the address arithmetic is scalar. These
//     loads carry the nontemporal hint: each instruction reads whole cache
//     lines that nothing reads again, and with the hint the gather runs ~9%
//     faster (the K loads, whose instructions touch 16 bytes of 64 lines
//     each, keep the default: the hint there re-fetches lines).
//   * scores: each lane dots its part of the row with the group's G query heads
//     (LDS broadcasts; v_dot2_f32_bf16 -- exact bf16 products, fp32 sums), and
//     row swaps (v_permlane16_swap, v_permlane32_swap) add the parts.
//   * online softmax in base 2 (the scale folds in log2 e) against a deferred
//     reference that is raised (one DPP wave max per head, and a rescale)
//     only when a score overtakes it by more than 2^8; the running sum stays
//     per lane and is reduced once at the end. Probabilities go to LDS.
//   * values: fp32 FMAs of the fp32 probabilities into per-lane accumulators.
// Padding slots (-1) may sit anywhere in a split (dsa_topk puts them at the
// end of a row): each has probability 0, the walk ends after the split's last
// valid slot, and an empty split writes o = 0, lse = -inf.

#include "dsa_kernels.h"

namespace dsa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSpan = 512;  // slots whose cache rows are resolved at once
constexpr float kSlack = 8.0f;  // log2 headroom of the deferred softmax reference

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Max over all 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Sum over all 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Orders this wave's LDS writes before its later LDS reads (the scratch it
// syncs on is private to the wave, so no workgroup barrier is needed).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Max over all 64 lanes of an int, wave-uniform.
__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// x[lane] + x[lane ^ 32] (N = 2: the two halves of a token's row in the
// vector kernel), or x summed over the four 16-lane rows (N = 4); every such
// lane gets the sum.
template <int N>
__device__ __forceinline__ float sum_token_lanes(float x) {
  if constexpr (N == 4) {
    const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                     false);
    x = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
  }
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// What one lane loads of a value row for its DPL output dims.
template <typename T, int DPL> struct Elem;
template <> struct Elem<uint16_t, 2> {
  typedef uint32_t Word;
  __device__ static float get(Word w, int i) {
    return i == 0 ? __uint_as_float(w << 16) : __uint_as_float(w & 0xFFFF0000u);
  }
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

// A value-row word loaded as streaming (nontemporal) data: the selected rows
// are read once, and the hint lets the gathers run closer to the streaming
// rate.
template <typename W> __device__ __forceinline__ W load_stream(const W* p) {
  return __builtin_nontemporal_load(p);
}
template <> __device__ __forceinline__ float2 load_stream<float2>(const float2* p) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  const f2v v = __builtin_nontemporal_load(reinterpret_cast<const f2v*>(p));
  return make_float2(v.x, v.y);
}

// FS == 0: one wave per workgroup and split, partials written to HBM.
// FS > 0: the FS splits of one (row, KV group) are FS waves of one workgroup
// and are merged through LDS into the final output (see the end); a
// workgroup holds PP such pairs (PP * FS waves), so that its waves can fill
// a CU's wave slots exactly (a workgroup's waves are all placed on one CU).
// Two lanes share a token (32-token tiles, each lane a half row).
template <typename T, int D, int G, int FS, int PP = 1>
__global__ __launch_bounds__(64 * (FS > 0 ? FS * PP : 1),
                             (sizeof(T) == 2 && D * G <= 1024) ? 3 : 2) void sparse_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ idx, int hkv, int k, int page_shift, int max_pages,
    float scale_log2, int S, int chunk, float* __restrict__ part_o,
    float* __restrict__ part_lse, void* __restrict__ out, float* __restrict__ out_lse,
    int npairs) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int RW = D * (int)sizeof(T) / 4;  // 32-bit words per row
  constexpr int LPT = 2;                      // lanes per token
  constexpr int TT = 64 / LPT;                // tokens per tile
  constexpr int NV4 = RW / 4 / LPT;           // uint4 per lane's part of a row
  constexpr int DPL = D / 64;                 // output dims per lane
  constexpr int NW = FS > 0 ? FS * PP : 1;    // waves per workgroup
  typedef Elem<T, DPL> E;
  typedef typename E::Word Word;
  __shared__ uint4 q_lds_all[PP][G * RW / 4];
  __shared__ float p_lds_all[NW][TT * G];
  __shared__ uint32_t rows_lds_all[NW][kSpan];

  const int lane = threadIdx.x & 63;
  // Uniform across the wave: everything derived from it (the pair, the
  // split, LDS slots, cache and index pointers) stays in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int tl = lane % TT, hf = lane / TT;  // token of the tile, part of its row
  // (row, KV group) pair of this wave; a workgroup's last pairs may not exist
  // (their waves skip the work but still meet the workgroup barriers).
  const int pw = FS > 0 ? wave / FS : 0;  // pair within the workgroup
  // Consecutive work items run on one XCD (workgroup i runs on XCD i % 8), so
  // the workgroups of a row, which read the same tokens' K/V blocks, share
  // that XCD's L2 and translation caches.
  const int wg = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
  const int pair = FS > 0 ? wg * PP + pw : wg / S;
  const bool live = FS == 0 || pair < npairs;
  const int g = (live ? pair : 0) % hkv;
  const int r = (live ? pair : 0) / hkv;
  const int s = FS > 0 ? wave - pw * FS : wg % S;
  const uint4* q_lds = q_lds_all[pw];
  float* p_lds = p_lds_all[wave];
  uint32_t* rows_lds = rows_lds_all[wave];
  const int hq = hkv * G;
  const int a = live ? min(k, s * chunk) : k;  // a dead pair's waves get an empty range
  const int b = min(k, a + chunk);
  const int page_mask = (1 << page_shift) - 1;
  const int32_t* btr = bt + (size_t)row_req[r] * max_pages;
  const int32_t* ir = idx + (size_t)r * k;
  const size_t kv_stride = (size_t)hkv * D;
  const T* kgroup = kc + (size_t)g * D;
  const T* vgroup = vc + (size_t)g * D;

  if (live) {
    // The FS waves of a pair load its query block together.
    const uint4* qsrc = reinterpret_cast<const uint4*>(q + ((size_t)r * hq + (size_t)g * G) * D);
    const int pt = threadIdx.x - pw * FS * 64;  // thread index within the pair
    for (int i = pt; i < G * RW / 4; i += 64 * (FS > 0 ? FS : 1)) q_lds_all[pw][i] = qsrc[i];
  }
  __syncthreads();  // every wave of the workgroup reads the whole query block

  float m[G], lsum[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.0f;
  }

  for (int c0 = a; c0 < b; c0 += kSpan) {
    const int n = min(b - c0, kSpan);
    // Resolve the span's selected positions to cache rows (0xFFFFFFFF for
    // padding) once, and find its last selected slot: every position load is
    // issued, then every block-table load, so the span costs two round trips.
    wave_sync();  // this wave's previous span readers are done with rows_lds
    constexpr int RPL = kSpan / 64;
    int pos[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int i = lane + 64 * u;
      pos[u] = i < n ? ir[c0 + i] : -1;
    }
    uint32_t prow[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u)
      prow[u] = pos[u] >= 0 ? (uint32_t)btr[pos[u] >> page_shift] : 0xFFFFFFFFu;
    int last = -1;
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int i = lane + 64 * u;
      const uint32_t row = pos[u] >= 0 ? ((prow[u] << page_shift) | (uint32_t)(pos[u] & page_mask))
                                       : 0xFFFFFFFFu;
      if (i < n) rows_lds[i] = row;
      if (pos[u] >= 0) last = i;
    }
    last = __builtin_amdgcn_readfirstlane(wave_max_i32(last));  // uniform: a scalar loop bound
    wave_sync();
    const int ntiles = (last + TT) / TT;  // tiles up to the last selected slot

    // Row ids of tile t for this lane's token (shared by its LPT lanes).
    auto tile_row = [&](int t) -> uint32_t {
      const int i = t * TT + tl;
      return i < n ? rows_lds[i] : 0xFFFFFFFFu;
    };
    // Loads are unconditional: a padding slot reads cache row 0 and gets
    // probability 0, so the load counters stay exact.
    auto load_k = [&](uint32_t row, uint4 (&kv)[NV4]) {
      const uint32_t rr = row == 0xFFFFFFFFu ? 0u : row;
      const uint4* kp = reinterpret_cast<const uint4*>(kgroup + (size_t)rr * kv_stride) + hf * NV4;
#pragma unroll
      for (int c = 0; c < NV4; ++c) kv[c] = kp[c];
    };

    uint32_t krow = tile_row(0);
    uint4 kv[NV4];
    load_k(krow, kv);
    for (int t = 0; t < ntiles; ++t) {
      // V of tile t: one whole row per token, its row id wave-uniform.
      Word vw[TT];
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        uint32_t rj = (uint32_t)__builtin_amdgcn_readlane((int)krow, j);
        rj = rj == 0xFFFFFFFFu ? 0u : rj;
        vw[j] = load_stream(reinterpret_cast<const Word*>(vgroup + (size_t)rj * kv_stride) + lane);
      }
      const bool valid = krow != 0xFFFFFFFFu;
      const uint32_t krow_next = tile_row(t + 1);

      // Scores for the group's heads (log2 units).
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4* qh = q_lds + h * (RW / 4) + hf * NV4;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < NV4; ++c) {
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
        sc[h] = valid ? sum_token_lanes<LPT>(acc) * scale_log2 : -INFINITY;
      }
      // K of tile t+1 in flight while tile t's values are summed.
      load_k(krow_next, kv);

      // Online softmax with a deferred reference: probabilities are taken
      // against the running reference m[h]; only when some score exceeds it
      // by more than 2^kSlack (or on the first tile, m = -inf) is the
      // reference raised to the true running max and the accumulators
      // rescaled. The result is the same normalized softmax -- o and the sum
      // share the reference -- and every probability stays <= 2^kSlack.
      bool over = false;
#pragma unroll
      for (int h = 0; h < G; ++h) over |= sc[h] > m[h] + kSlack;
      if (__ballot(over) != 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mn = fmaxf(m[h], wave_max(sc[h]));
          const float alpha = fast_exp2(m[h] - mn);  // m = -inf: alpha = 0
          lsum[h] *= alpha;
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[h][e] *= alpha;
          m[h] = mn;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // A padding slot has probability 0 whatever the reference: before the
        // split's first valid slot m is still -inf, and -inf - -inf is NaN.
        const float p = valid ? fast_exp2(sc[h] - m[h]) : 0.0f;
        lsum[h] += (hf == 0) ? p : 0.0f;
        if (hf == 0) p_lds[tl * G + h] = p;
      }
      wave_sync();

#pragma unroll
      for (int j = 0; j < TT; ++j) {
        float pj[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pj[h] = p_lds[j * G + h];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[h][e] = fmaf(pj[h], E::get(vw[j], e), o[h][e]);
      }
      wave_sync();
      krow = krow_next;
    }
  }

  if constexpr (FS == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float l = wave_sum(lsum[h]);
      const size_t head = (size_t)r * hq + (size_t)g * G + h;
      const bool any = l > 0.0f;
      const float inv = any ? 1.0f / l : 0.0f;
      float* po = part_o + (head * S + s) * D + (size_t)lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) po[e] = o[h][e] * inv;
      if (lane == 0) part_lse[head * S + s] = any ? (m[h] + __log2f(l)) * kLn2 : -INFINITY;
    }
  } else {
    // The FS split partials go to LDS (the same values the unfused kernel
    // writes to HBM) and are merged exactly as dsa_merge does -- same
    // operations in the same split order -- so both paths agree bit for bit.
    __shared__ float o_lds[NW][G][D];
    __shared__ float lse_lds[NW][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float l = wave_sum(lsum[h]);
      const bool any = l > 0.0f;
      const float inv = any ? 1.0f / l : 0.0f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o_lds[wave][h][lane * DPL + e] = o[h][e] * inv;
      if (lane == 0) lse_lds[wave][h] = any ? (m[h] + __log2f(l)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < PP * G * D; i += 64 * NW) {
      const int pp = i / (G * D);
      const int hd = i - pp * G * D;
      const int h = hd / D, e = hd - h * D;
      const int pr = wg * PP + pp;
      if (pr >= npairs) break;  // the pairs past the end come last
      const int r = pr / hkv, g = pr - r * hkv;
      const int w0 = pp * FS;
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < FS; ++u) M = fmaxf(M, lse_lds[w0 + u][h]);
      const bool any = M != -INFINITY;
      const float Mr = any ? M : 0.0f;
      float W = 0.0f, acc = 0.0f;
#pragma unroll
      for (int u = 0; u < FS; ++u) {
        const float wgt = __expf(lse_lds[w0 + u][h] - Mr);
        W += wgt;
        acc = fmaf(wgt, o_lds[w0 + u][h][e], acc);
      }
      const float invW = any ? 1.0f / W : 0.0f;
      const float x = acc * invW;
      const size_t oi = ((size_t)r * hq + (size_t)g * G + h) * D + e;
      if constexpr (kBf16) static_cast<uint16_t*>(out)[oi] = f32_to_bf16_rne(x);
      else static_cast<float*>(out)[oi] = x;
      if (out_lse && e == 0) out_lse[(size_t)r * hq + (size_t)g * G + h] = any ? M + __logf(W) : -INFINITY;
    }
  }
}

// Matrix-core tiles for bf16 rows, d = 128, eight query heads per KV group
// (the decode shape of the method's models). The vector kernel above spends
// most of its issue slots on the dot products and the value FMAs; here both
// contractions run on v_mfma and the vector unit keeps only the softmax:
//   * copies: tile t's K and V rows go straight from global memory to the
//     wave's LDS buffers (global_load_lds): each instruction takes four
//     tokens' whole 256-byte rows, which reads the gathered rows ~10% faster
//     than quarter rows per token (with the top-k's positions shared by a
//     row's KV groups, as here);
//   * scores S^T[16 tokens x 16 heads] = K[16 x 128] . Q^T (v_mfma_f32_16x16x32_bf16,
//     four steps): lane l reads the K fragments of token l % 16, dims
//     32 (l / 16) .. + 32, from LDS and the query fragments of head l % 16
//     (heads 8..15 are zero columns); the result gives lane l head l % 16 at
//     tokens 4 (l / 16) .. + 4 -- exactly the layout of P^T as the B operand
//     of the value product, so the probabilities never leave registers;
//   * values O^T[128 x 16 heads] += V^T . P^T with V read transposed out of
//     LDS (ds_read_b64_tr_b16); the fp32 probabilities are split exactly
//     into three bf16 terms (hi + mid + lo: a float's 24 significand bits),
//     each multiplied with V in a 16x16x16 product and summed in fp32, so the
//     value reduction keeps the fp32 probabilities;
//   * one tile in flight: once tile t's K fragments are in registers, tile
//     t + 1's K rows are copied into the same buffer; once its V fragments
//     are (after the softmax), tile t + 1's V rows; both land while tile t
//     is computed.
// Splits, spans, padding, the deferred softmax reference and the merged
// epilogue are those of the vector kernel.
namespace {
typedef __bf16 mx_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mx_bf16x4 __attribute__((ext_vector_type(4)));
typedef short mx_i16x4 __attribute__((ext_vector_type(4)));
typedef float mx_f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void mx_gvoid;
typedef __attribute__((address_space(3))) void mx_lvoid;
typedef __attribute__((address_space(3))) mx_bf16x4 mx_lds_bf16x4;
constexpr int kMxTile = 16;   // tokens per tile
// s_waitcnt immediate (gfx9 encoding): no vector memory instruction
// outstanding; LDS, scalar and export counters not waited on.
constexpr int kMxWaitVm0 = 0 | (7 << 4) | (15 << 8);
// No LDS (or scalar memory) instruction outstanding; vector memory not waited on.
constexpr int kMxWaitLgkm0 = 15 | (3 << 14) | (7 << 4);
}  // namespace

// Piece p (16 bytes, 8 dims) of token j's row sits in LDS slot p ^ f(j), so
// that the 16 tokens of one fragment read land on distinct bank groups: for K
// (16-byte reads of piece 4 (l / 16) + c of token l % 16) f(j) = j % 16, for
// V (transposing 8-byte reads, four tokens x four dims per 16-lane group)
// f(j) = 2 (j % 8).
__device__ __forceinline__ int mx_kslot(int j) { return j & 15; }
__device__ __forceinline__ int mx_vslot(int j) { return (j & 7) << 1; }

// Max over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float max_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Orders memory operations around an explicit wait (compiler and scheduler).
__device__ __forceinline__ void mx_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int FS, int PP = 1>
__global__ __launch_bounds__(64 * (FS > 0 ? FS * PP : 1), 4) void sparse_attn_mx_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ row_req, const int32_t* __restrict__ idx, int hkv, int k,
    int page_shift, int max_pages, float scale_log2, int S, int chunk,
    float* __restrict__ part_o, float* __restrict__ part_lse, void* __restrict__ out,
    float* __restrict__ out_lse, int npairs) {
  constexpr int D = 128, G = 8;
  constexpr int NW = FS > 0 ? FS * PP : 1;  // waves per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[NW][kMxTile * D];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[NW][kMxTile * D];
  // Slots resolved to cache rows at once: a whole split up to 512 (one
  // prologue per wave at four splits of 2048), 256 in 16-wave workgroups
  // (the LDS holds no more).
  constexpr int SPAN = NW <= 8 ? 512 : 256;
  constexpr int RPL = SPAN / 64;
  __shared__ uint32_t rows_all[NW][SPAN];
  // Each pair's query block as 16 head rows (rows G..15 zero: the padding
  // columns of the score tiles), rows padded so a fragment read spreads over
  // the banks.
  constexpr int QST = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t q_lds_all[PP][16 * QST];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int tl = lane & 15, hf = lane >> 4;  // token (K, scores) or head (P, O) / row group
  const int pw = FS > 0 ? wave / FS : 0;
  const int wg = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
  const int pair = FS > 0 ? wg * PP + pw : wg / S;
  const bool live = FS == 0 || pair < npairs;
  const int g = (live ? pair : 0) % hkv;
  const int r = (live ? pair : 0) / hkv;
  const int s = FS > 0 ? wave - pw * FS : wg % S;
  uint32_t* rows_lds = rows_all[wave];
  uint16_t* kb = kbuf[wave];
  uint16_t* vb = vbuf[wave];
  const int hq = hkv * G;
  const int a = live ? min(k, s * chunk) : k;
  const int b = min(k, a + chunk);
  const int page_mask = (1 << page_shift) - 1;
  const int32_t* btr = bt + (size_t)row_req[r] * max_pages;
  const int32_t* ir = idx + (size_t)r * k;
  const uint32_t kv_stride = (uint32_t)hkv * D;  // elements per cache row (one 32x32->64 product per address)
  const uint16_t* kgroup = kc + (size_t)g * D;
  const uint16_t* vgroup = vc + (size_t)g * D;
  const bool head_lane = tl < G;

  // The first span's selected positions are requested before the query
  // block, so that the two loads' latencies overlap.
  int pos[RPL];
  auto load_pos = [&](int c0, int n) {
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int i = lane + 64 * u;
      pos[u] = i < n ? ir[c0 + i] : -1;
    }
  };
  load_pos(a, min(b - a, SPAN));

  // The waves of a pair load its query block together (a dead pair's waves
  // write zeros).
  {
    const int pt = threadIdx.x - pw * (FS > 0 ? FS : 1) * 64;  // thread within the pair
    const uint4* qsrc = reinterpret_cast<const uint4*>(q + ((size_t)r * hq + (size_t)g * G) * D);
    for (int i = pt; i < 16 * D / 8; i += 64 * (FS > 0 ? FS : 1)) {
      const int h = i / (D / 8), c = i - h * (D / 8);
      const uint4 v = (live && h < G) ? qsrc[h * (D / 8) + c] : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&q_lds_all[pw][h * QST + c * 8]) = v;
    }
  }
  __syncthreads();
  // Query fragments of step c: head tl, dims 32 hf + 8 c .. + 8.
  const uint16_t* qfrag = &q_lds_all[pw][tl * QST + hf * 32];

  float m = -INFINITY, lsum = 0.0f;  // head tl's reference and this lane's part of its sum
  mx_f32x4 o[D / 16];                 // O^T: head tl, dims 16 nt + 4 hf .. + 4
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) o[nt] = mx_f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int c0 = a; c0 < b; c0 += SPAN) {
    const int n = min(b - c0, SPAN);
    wave_sync();  // this wave's previous span readers are done with rows_lds
    if (c0 != a) load_pos(c0, n);
    uint32_t prow[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u)
      prow[u] = pos[u] >= 0 ? (uint32_t)btr[pos[u] >> page_shift] : 0xFFFFFFFFu;
    int last = -1;
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int i = lane + 64 * u;
      const uint32_t row = pos[u] >= 0 ? ((prow[u] << page_shift) | (uint32_t)(pos[u] & page_mask))
                                       : 0xFFFFFFFFu;
      if (i < n) rows_lds[i] = row;
      if (pos[u] >= 0) last = i;
    }
    last = __builtin_amdgcn_readfirstlane(wave_max_i32(last));
    wave_sync();
    const int ntiles = (last + kMxTile) / kMxTile;

    auto row_of = [&](int i) -> uint32_t { return i < n ? rows_lds[i] : 0xFFFFFFFFu; };
    // Row ids of the tokens whose rows this lane copies for tile t (tokens
    // 4u + l / 16); padding copies cache row 0 (probability 0), so every
    // copy is issued.
    auto tile_rows = [&](int t, uint32_t (&rr)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t row = row_of(t * kMxTile + 4 * u + hf);
        rr[u] = row == 0xFFFFFFFFu ? 0u : row;
      }
    };
    // Instruction u copies tokens 4u .. 4u + 3: lane l takes piece
    // (l % 16) ^ f(token) of token 4u + l / 16, which lands in slot l % 16 of
    // that token's 256 bytes.
    auto copy_k = [&](const uint32_t (&rr)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_global_load_lds(
            (mx_gvoid*)(kgroup + (uint64_t)rr[u] * kv_stride + 8 * (tl ^ mx_kslot(4 * u + hf))),
            (mx_lvoid*)(kb + u * 4 * D), 16, 0, 0);
    };
    auto copy_v = [&](const uint32_t (&rr)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_global_load_lds(
            (mx_gvoid*)(vgroup + (uint64_t)rr[u] * kv_stride + 8 * (tl ^ mx_vslot(4 * u + hf))),
            (mx_lvoid*)(vb + u * 4 * D), 16, 0, 0);
    };

    uint32_t rr[4];
    if (ntiles > 0) {
      tile_rows(0, rr);
      copy_k(rr);
      copy_v(rr);
    }
    // Fragment read addresses: K piece 4 hf + c of token tl; V dims
    // 16 nt + 4 (j % 4) .. + 4 of token 4 hf + j / 4 for lane j of a 16-lane
    // group (the transposing read then gives lane m dim 16 nt + m of the four
    // tokens 4 hf .. + 4).
    const uint16_t* kfrag = kb + tl * D;
    const int tv = 4 * hf + (tl >> 2);
    const uint16_t* vrow = vb + tv * D;
    for (int t = 0; t < ntiles; ++t) {
      __builtin_amdgcn_s_waitcnt(kMxWaitVm0);  // tile t's copies have landed
      mx_fence();
      mx_bf16x8 ka[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        ka[c] = *reinterpret_cast<const mx_bf16x8*>(kfrag + 8 * ((4 * hf + c) ^ mx_kslot(tl)));
      const uint32_t trow = row_of(t * kMxTile + tl);
      const bool more = t + 1 < ntiles;
      if (more) tile_rows(t + 1, rr);
      // The K fragments are in registers: tile t + 1's K rows may reuse the buffer.
      __builtin_amdgcn_s_waitcnt(kMxWaitLgkm0);
      mx_fence();
      if (more) copy_k(rr);
      const uint32_t vmask = (uint32_t)__ballot(trow != 0xFFFFFFFFu) & 0xFFFFu;

      // The query fragments are read per tile: the empty asm makes their
      // address opaque, so they are not hoisted into 16 loop-long registers.
      int qoff = 0;
      asm volatile("" : "+v"(qoff));
      mx_f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            ka[c], *reinterpret_cast<const mx_bf16x8*>(qfrag + qoff + c * 8), sc, 0, 0, 0);
      bool ok[4];
      float sv[4];
      bool over = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[i] = head_lane && ((vmask >> (4 * hf + i)) & 1u);
        sv[i] = ok[i] ? sc[i] * scale_log2 : -INFINITY;
        over |= sv[i] > m + kSlack;
      }
      // Deferred reference (as in the vector kernel): raised to the running
      // max, with a rescale, only when a score overtakes it by 2^kSlack.
      if (__ballot(over) != 0) {
        const float mx = max_rows4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        const float mn = fmaxf(m, mx);
        const float alpha = m == mn ? 1.0f : fast_exp2(m - mn);  // m = -inf: 0
        lsum *= alpha;
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) o[nt] *= alpha;
        m = mn;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = ok[i] ? fast_exp2(sv[i] - m) : 0.0f;
      lsum += (p[0] + p[1]) + (p[2] + p[3]);

      // p = hi + mid + lo exactly, each a bf16 (truncations of the remainder).
      uint32_t hb[4], mb[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u0 = __float_as_uint(p[i]);
        const float r1 = p[i] - __uint_as_float(u0 & 0xFFFF0000u);  // exact
        const uint32_t u1 = __float_as_uint(r1);
        const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);    // exact, <= 8 bits
        hb[i] = u0 >> 16;
        mb[i] = u1 >> 16;
        lb[i] = __float_as_uint(r2) >> 16;
      }
      // B operands of v_mfma_f32_16x16x16_bf16: k index 4 hf + e is token
      // 4 hf + e, one product per term. (All three products have one shape: a
      // 16x16x16 product issued right after a 16x16x32 one on the same
      // accumulator read part of it stale on this hardware -- rows 4 hf and
      // 4 hf + 1 lost the first product -- while products of one shape chain.)
      const mx_i16x4 phi = __builtin_bit_cast(mx_i16x4, make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)));
      const mx_i16x4 pmi = __builtin_bit_cast(mx_i16x4, make_uint2(mb[0] | (mb[1] << 16), mb[2] | (mb[3] << 16)));
      const mx_i16x4 plo = __builtin_bit_cast(mx_i16x4, make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)));
      // V^T fragments, then tile t + 1's V rows into the buffer they leave.
      mx_bf16x4 vt[D / 16];
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        const int d0 = nt * 16 + 4 * (tl & 3);
        const uint16_t* src = vrow + 8 * ((d0 >> 3) ^ mx_vslot(tv)) + (d0 & 7);
        vt[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (mx_lds_bf16x4*)(__attribute__((address_space(3))) uint16_t*)src);
      }
      __builtin_amdgcn_s_waitcnt(kMxWaitLgkm0);
      mx_fence();
      if (more) copy_v(rr);
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        const mx_i16x4 v = __builtin_bit_cast(mx_i16x4, vt[nt]);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, phi, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pmi, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, plo, o[nt], 0, 0, 0);
      }
    }
  }

  // Head tl's sum over the four row groups (every such lane gets it).
  const float l = sum_token_lanes<4>(lsum);
  const bool any = l > 0.0f;
  const float inv = any ? 1.0f / l : 0.0f;
  if constexpr (FS == 0) {
    if (head_lane) {
      const size_t head = (size_t)r * hq + (size_t)g * G + tl;
      float* po = part_o + (head * S + s) * D + 4 * hf;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt)
        *reinterpret_cast<float4*>(po + nt * 16) =
            make_float4(o[nt][0] * inv, o[nt][1] * inv, o[nt][2] * inv, o[nt][3] * inv);
      if (hf == 0) part_lse[head * S + s] = any ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
  } else {
    // The split partials go to LDS over this wave's V buffer (its copies
    // have all landed: each tile waits for everything requested, and the
    // last tile requests nothing), then merge as dsa_merge does.
    __shared__ float lse_lds[NW][G];
    float* o_w = reinterpret_cast<float*>(vb);  // [G][D]
    wave_sync();
    if (head_lane) {
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt)
        *reinterpret_cast<float4*>(o_w + tl * D + nt * 16 + 4 * hf) =
            make_float4(o[nt][0] * inv, o[nt][1] * inv, o[nt][2] * inv, o[nt][3] * inv);
      if (hf == 0) lse_lds[wave][tl] = any ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < PP * G * D; i += 64 * NW) {
      const int pp = i / (G * D);
      const int hd = i - pp * G * D;
      const int h = hd / D, e = hd - h * D;
      const int pr = wg * PP + pp;
      if (pr >= npairs) break;  // the pairs past the end come last
      const int r2 = pr / hkv, g2 = pr - r2 * hkv;
      const int w0 = pp * FS;
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < FS; ++u) M = fmaxf(M, lse_lds[w0 + u][h]);
      const bool anyw = M != -INFINITY;
      const float Mr = anyw ? M : 0.0f;
      float W = 0.0f, acc = 0.0f;
#pragma unroll
      for (int u = 0; u < FS; ++u) {
        const float wgt = __expf(lse_lds[w0 + u][h] - Mr);
        W += wgt;
        acc = fmaf(wgt, reinterpret_cast<const float*>(vbuf[w0 + u])[h * D + e], acc);
      }
      const float invW = anyw ? 1.0f / W : 0.0f;
      const float x = acc * invW;
      const size_t oi = ((size_t)r2 * hq + (size_t)g2 * G + h) * D + e;
      static_cast<uint16_t*>(out)[oi] = f32_to_bf16_rne(x);
      if (out_lse && e == 0) out_lse[(size_t)r2 * hq + (size_t)g2 * G + h] = anyw ? M + __logf(W) : -INFINITY;
    }
  }
}

// The shape that runs on the matrix-core kernel (bf16, d = 128, eight query
// heads per KV group). The choice depends only on the shape, so the merged
// and two-launch paths of one call use the same kernel and stay bitwise equal.
template <typename T, int D, int G>
constexpr bool mx_shape() {
  return sizeof(T) == 2 && D == 128 && G == 8;
}

template <typename T, int FS, int PP = 1>
static hipError_t launch_attn_t(const T* q, const T* kc, const T* vc, const int32_t* bt,
                                const int32_t* row_req, const int32_t* idx, int rows, int hq,
                                int hkv, int d, int k, int page_shift, int max_pages, float scale,
                                int S, float* part_o, float* part_lse, void* out, float* out_lse,
                                hipStream_t stream) {
  const int G = hq / hkv;
  const int chunk = (k + S - 1) / S;
  const int npairs = rows * hkv;
  const dim3 grid(FS > 0 ? (unsigned)((npairs + PP - 1) / PP) : (unsigned)rows * S * hkv);
  const dim3 block(64 * (FS > 0 ? FS * PP : 1));
  const float sl2 = scale * kLog2e;
#define DSA_ATTN(D_, G_)                                                                       \
  if constexpr (mx_shape<T, D_, G_>())                                                         \
    hipLaunchKernelGGL((sparse_attn_mx_kernel<FS, PP>), grid, block, 0, stream,                \
                       reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(kc), \
                       reinterpret_cast<const uint16_t*>(vc), bt, row_req, idx, hkv, k,         \
                       page_shift, max_pages, sl2, S, chunk, part_o, part_lse, out, out_lse,    \
                       npairs);                                                                \
  else                                                                                         \
    hipLaunchKernelGGL((sparse_attn_kernel<T, D_, G_, FS, PP>), grid, block, 0, stream, q, kc,  \
                       vc, bt, row_req, idx, hkv, k, page_shift, max_pages, sl2, S, chunk,      \
                       part_o, part_lse, out, out_lse, npairs)
#define DSA_ATTN_G(D_)                    \
  switch (G) {                            \
    case 1: DSA_ATTN(D_, 1); break;       \
    case 2: DSA_ATTN(D_, 2); break;       \
    case 4: DSA_ATTN(D_, 4); break;       \
    case 8: DSA_ATTN(D_, 8); break;       \
    case 16: DSA_ATTN(D_, 16); break;     \
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

template <typename T>
static const void* attn_kernel_ptr(int d, int G) {
#define DSA_ATTN_PTR(D_, G_)                                                               \
  if (d == D_ && G == G_) {                                                                \
    if constexpr (mx_shape<T, D_, G_>()) return (const void*)sparse_attn_mx_kernel<0, 1>;  \
    else return (const void*)sparse_attn_kernel<T, D_, G_, 0, 1>;                         \
  }
  DSA_ATTN_PTR(128, 1) DSA_ATTN_PTR(128, 2) DSA_ATTN_PTR(128, 4) DSA_ATTN_PTR(128, 8)
  DSA_ATTN_PTR(128, 16) DSA_ATTN_PTR(64, 1) DSA_ATTN_PTR(64, 2) DSA_ATTN_PTR(64, 4)
  DSA_ATTN_PTR(64, 8) DSA_ATTN_PTR(64, 16)
#undef DSA_ATTN_PTR
  return nullptr;
}

int attn_default_splits(int rows, int hq, int hkv, int d, int k, bool bf16) {
  const long long pairs = (long long)rows * hkv;
  const void* kern = bf16 ? attn_kernel_ptr<uint16_t>(d, hq / hkv)
                          : attn_kernel_ptr<float>(d, hq / hkv);
  int cap = kern ? device_capacity(kern, 64) : 0;
  if (cap <= 0) cap = 3072;
  // Waves of one launch ~ two thirds of the device's capacity: longer waves
  // amortize their prologue (query load, position -> row resolution) better
  // than a full first round does; each split keeps >= 32 slots.
  const long long waves = pairs;
  const long long target = 2LL * cap / 3;
  int s = (int)((target + waves / 2) / waves);
  const int max_s = max(1, k / 32);
  return max(1, min(s, max_s));
}

hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* bt,
                              const int32_t* row_req, const int32_t* idx, int rows, int hq,
                              int hkv, int d, int k, int page_shift, int max_pages, float scale,
                              int num_splits, float* part_o, float* part_lse, bool bf16,
                              hipStream_t stream) {
  if (bf16)
    return launch_attn_t<uint16_t, 0>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
        static_cast<const uint16_t*>(vc), bt, row_req, idx, rows, hq, hkv, d, k, page_shift,
        max_pages, scale, num_splits, part_o, part_lse, nullptr, nullptr, stream);
  return launch_attn_t<float, 0>(static_cast<const float*>(q), static_cast<const float*>(kc),
                                 static_cast<const float*>(vc), bt, row_req, idx, rows, hq, hkv, d,
                                 k, page_shift, max_pages, scale, num_splits, part_o, part_lse,
                                 nullptr, nullptr, stream);
}

// Eight splits of the matrix-core shape: two (row, KV group) pairs per
// 16-wave workgroup fill a CU at four waves per SIMD.
static hipError_t launch_merged_mx8(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                                   const int32_t* bt, const int32_t* row_req, const int32_t* idx,
                                   int rows, int hkv, int k, int page_shift, int max_pages,
                                   float scale, void* out, float* out_lse, hipStream_t stream) {
  constexpr int kS = 8, kPP = 2;
  const int npairs = rows * hkv;
  const int chunk = (k + kS - 1) / kS;
  hipLaunchKernelGGL((sparse_attn_mx_kernel<kS, kPP>),
                     dim3((unsigned)((npairs + kPP - 1) / kPP)), dim3(64 * kS * kPP), 0, stream, q,
                     kc, vc, bt, row_req, idx, hkv, k, page_shift, max_pages, scale * kLog2e, kS,
                     chunk, nullptr, nullptr, out, out_lse, npairs);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_merged_t(const void* q, const void* kc, const void* vc, const int32_t* bt,
                                  const int32_t* row_req, const int32_t* idx, int rows, int hq,
                                  int hkv, int d, int k, int page_shift, int max_pages, float scale,
                                  int S, void* out, float* out_lse, hipStream_t stream) {
  const T* q_ = static_cast<const T*>(q);
  const T* k_ = static_cast<const T*>(kc);
  const T* v_ = static_cast<const T*>(vc);
#define DSA_MERGED(FS_, PP_)                                                                   \
  return launch_attn_t<T, FS_, PP_>(q_, k_, v_, bt, row_req, idx, rows, hq, hkv, d, k,          \
                                    page_shift, max_pages, scale, S, nullptr, nullptr, out,     \
                                    out_lse, stream)
  // Six splits run as two (row, KV group) pairs per workgroup: twelve waves
  // fill a CU's wave slots at three waves per SIMD, where a six-wave
  // workgroup would leave half of them empty.
  // (fp32 rows keep one pair per workgroup: two would exceed the LDS.)
  constexpr int kPairs6 = sizeof(T) == 2 ? 2 : 1;
  switch (S) {
    case 1: DSA_MERGED(1, 1);
    case 2: DSA_MERGED(2, 1);
    case 4:
      // On the matrix-core kernel two pairs (8 waves, 82 KB of LDS) take a
      // CU each, which spreads a batch of 2 x CUs pairs evenly (~1% faster
      // than one pair per workgroup, where some CUs hold three).
      if (sizeof(T) == 2 && d == 128 && hq == 8 * hkv) DSA_MERGED(4, 2);
      DSA_MERGED(4, 1);
    case 6: DSA_MERGED(6, kPairs6);
    case 8:
      // On the matrix-core kernel two pairs (16 waves) fit a workgroup.
      if (sizeof(T) == 2 && d == 128 && hq == 8 * hkv)
        return launch_merged_mx8(reinterpret_cast<const uint16_t*>(q_),
                                reinterpret_cast<const uint16_t*>(k_),
                                 reinterpret_cast<const uint16_t*>(v_), bt, row_req, idx, rows, hkv,
                                 k, page_shift, max_pages, scale, out, out_lse, stream);
      DSA_MERGED(8, 1);
    default: return hipErrorInvalidValue;
  }
#undef DSA_MERGED
}

hipError_t launch_sparse_attn_merged(const void* q, const void* kc, const void* vc,
                                     const int32_t* bt, const int32_t* row_req, const int32_t* idx,
                                     int rows, int hq, int hkv, int d, int k, int page_shift,
                                     int max_pages, float scale, int num_splits, void* out,
                                     float* out_lse, bool bf16, hipStream_t stream) {
  if (bf16)
    return launch_merged_t<uint16_t>(q, kc, vc, bt, row_req, idx, rows, hq, hkv, d, k, page_shift,
                                     max_pages, scale, num_splits, out, out_lse, stream);
  return launch_merged_t<float>(q, kc, vc, bt, row_req, idx, rows, hq, hkv, d, k, page_shift,
                                max_pages, scale, num_splits, out, out_lse, stream);
}

int merged_default_splits(int rows, int hq, int hkv, int d, int k, bool bf16) {
  // Vector kernel: six splits in workgroups of two pairs when that fills the
  // device in about one round at three waves per SIMD (the rows x KV groups
  // are many, the occupancy allows it); otherwise the split kernel's
  // suggestion rounded down to a supported workgroup size (1, 2, 4 or 8
  // waves).
  const long long pairs = (long long)rows * hkv;
  const void* kern = bf16 ? attn_kernel_ptr<uint16_t>(d, hq / hkv)
                          : attn_kernel_ptr<float>(d, hq / hkv);
  int cus = device_cus();
  int cap = kern ? device_capacity(kern, 64) : 0;
  if (cap <= 0 || cus <= 0) {
    cus = 256;
    cap = 3072;
  }
  if (bf16 && d == 128 && hq == 8 * hkv) {
    // Matrix-core kernel: the fewest splits (the longest walk per wave, each
    // wave paying the position -> row prologue and its share of the merge
    // once) that still put about seven waves on every CU. At 64 rows x 8
    // groups four splits (8 waves per CU) run ~4% faster than six or eight;
    // two (4 waves per CU) run 35% slower.
    int s = 1;
    while (s < 8 && pairs * s < 7LL * cus) s *= 2;
    while (s > 1 && s * 16 > k) s /= 2;  // at least one 16-token tile per split
    return s;
  }
  if (cap / cus == 12 && k >= 6 * 32 && pairs * 6 <= cap && pairs * 6 * 2 >= cap) return 6;
  const int s = attn_default_splits(rows, hq, hkv, d, k, bf16);
  int f = 1;
  while (f * 2 <= s && f * 2 <= 8 && f * 2 <= k) f *= 2;
  return f;
}

}  // namespace dsa
