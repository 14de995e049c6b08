// GQA sparse attention over split k-slot slices (Megatron-LM pull request
// 7211, commit "Replace the CuTe decode kernels with two Triton kernels": one
// program handles all query heads of a KV group, reading each selected key and
// value once, and the top-k slots are split across programs; commit "Restore
// the upstream Blackwell FP32 probability reduction": probabilities stay fp32
// through the value reduction).
//
// One wave per (row, split, KV group); in the merged variant the splits of one
// (row, KV group) are the waves of one workgroup and are merged through LDS at
// the end (no partials in HBM, no second launch). The split's slots are walked
// in tiles of 32 tokens (two lanes per token) or 16 (four lanes per token):
//   * addresses: a prologue translates up to 512 selected positions through
//     the block table into cache row ids in LDS (two dependent round trips
//     per span, not per tile); tiles past the span's last selected slot are
//     skipped.
//   * pipelining: V of tile t is requested before tile t's scores, K of tile
//     t+1 before tile t's value sums; every load is unconditional (padding
//     reads cache row 0 with probability 0), so each wait covers exactly the
//     data in use.
//   * K: lane t reads the first half of token t's row for the group, lane
//     t + 32 the second half (two 128-byte runs per 256-byte bf16 row); with
//     16-token tiles lanes t, t+16, t+32, t+48 read its quarters.
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

// x summed over the LPT lanes of a token: x[lane] + x[lane ^ 32] (LPT 2), or
// over the four 16-lane rows (LPT 4); every such lane gets the sum.
template <int LPT>
__device__ __forceinline__ float sum_token_lanes(float x) {
  if constexpr (LPT == 4) {
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
// LPT lanes share a token: 2 (32-token tiles, each lane a half row) or 4
// (16-token tiles, quarter rows: fewer registers in flight per wave, so four
// waves fit a SIMD).
template <typename T, int D, int G, int FS, int PP = 1, int LPT = 2>
__global__ __launch_bounds__(64 * (FS > 0 ? FS * PP : 1),
                             LPT == 4 ? 4 : (sizeof(T) == 2 && D * G <= 1024) ? 3 : 2) void sparse_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ idx, int hkv, int k, int page_shift, int max_pages,
    float scale_log2, int S, int chunk, float* __restrict__ part_o,
    float* __restrict__ part_lse, void* __restrict__ out, float* __restrict__ out_lse,
    int npairs) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int RW = D * (int)sizeof(T) / 4;  // 32-bit words per row
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

// Lanes per token. bf16 rows with d = 128 and eight query heads per KV group
// (the decode shape of the method's models) can take 16-token tiles: 120
// registers, so four waves share a SIMD where 32-token tiles (168) allow
// three. That hides load latency in batches of up to a few waves per SIMD
// (~6% faster at batch 64); past that the kernel is bound by its vector
// arithmetic, which 32-token tiles spend less of per token. The choice
// depends only on the shape and rows x KV groups, so the merged and
// two-launch paths of one call shape use the same tiles and stay bitwise
// equal.
template <typename T, int D, int G>
constexpr bool quarter_tiles_shape() {
  return sizeof(T) == 2 && D == 128 && G == 8;
}
static bool quarter_tiles(bool shape_ok, long long pairs) {
  return shape_ok && pairs <= 8LL * device_cus();
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
#define DSA_ATTN_L(D_, G_, L_)                                                                  \
  hipLaunchKernelGGL((sparse_attn_kernel<T, D_, G_, FS, PP, L_>), grid, block, 0, stream, q, kc,  \
                     vc, bt, row_req, idx, hkv, k, page_shift, max_pages, sl2, S, chunk, part_o,  \
                     part_lse, out, out_lse, npairs)
#define DSA_ATTN(D_, G_)                                                       \
  if constexpr (quarter_tiles_shape<T, D_, G_>()) {                            \
    if (quarter_tiles(true, npairs)) DSA_ATTN_L(D_, G_, 4);                    \
    else DSA_ATTN_L(D_, G_, 2);                                                \
  } else {                                                                     \
    DSA_ATTN_L(D_, G_, 2);                                                     \
  }
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
#undef DSA_ATTN_L
  return hipGetLastError();
}

template <typename T>
static const void* attn_kernel_ptr(int d, int G, long long pairs) {
#define DSA_ATTN_PTR(D_, G_)                                                               \
  if (d == D_ && G == G_) {                                                                \
    if (quarter_tiles(quarter_tiles_shape<T, D_, G_>(), pairs))                              \
      return (const void*)sparse_attn_kernel<T, D_, G_, 0, 1, quarter_tiles_shape<T, D_, G_>() ? 4 : 2>; \
    return (const void*)sparse_attn_kernel<T, D_, G_, 0, 1, 2>;                           \
  }
  DSA_ATTN_PTR(128, 1) DSA_ATTN_PTR(128, 2) DSA_ATTN_PTR(128, 4) DSA_ATTN_PTR(128, 8)
  DSA_ATTN_PTR(128, 16) DSA_ATTN_PTR(64, 1) DSA_ATTN_PTR(64, 2) DSA_ATTN_PTR(64, 4)
  DSA_ATTN_PTR(64, 8) DSA_ATTN_PTR(64, 16)
#undef DSA_ATTN_PTR
  return nullptr;
}

int attn_default_splits(int rows, int hq, int hkv, int d, int k, bool bf16) {
  const long long pairs = (long long)rows * hkv;
  const void* kern = bf16 ? attn_kernel_ptr<uint16_t>(d, hq / hkv, pairs)
                          : attn_kernel_ptr<float>(d, hq / hkv, pairs);
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

// Eight splits of the 16-token-tile shape: two (row, KV group) pairs per
// 16-wave workgroup fill a CU at four waves per SIMD.
static hipError_t launch_merged_q4(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                                   const int32_t* bt, const int32_t* row_req, const int32_t* idx,
                                   int rows, int hkv, int k, int page_shift, int max_pages,
                                   float scale, void* out, float* out_lse, hipStream_t stream) {
  constexpr int kS = 8, kPP = 2;
  const int npairs = rows * hkv;
  const int chunk = (k + kS - 1) / kS;
  hipLaunchKernelGGL((sparse_attn_kernel<uint16_t, 128, 8, kS, kPP, 4>),
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
    case 4: DSA_MERGED(4, 1);
    case 6: DSA_MERGED(6, kPairs6);
    case 8:
      // With 16-token tiles two pairs (16 waves) fit a workgroup.
      if (quarter_tiles(sizeof(T) == 2 && d == 128 && hq == 8 * hkv, (long long)rows * hkv))
        return launch_merged_q4(reinterpret_cast<const uint16_t*>(q_),
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
  // Eight splits (16-token tiles) or six (32-token tiles) in workgroups of
  // two pairs when that fills the device in about one round at four or three
  // waves per SIMD (the rows x KV groups are many, the occupancy allows it);
  // otherwise the split kernel's suggestion rounded down to a supported
  // workgroup size (1, 2, 4 or 8 waves).
  const long long pairs = (long long)rows * hkv;
  const void* kern = bf16 ? attn_kernel_ptr<uint16_t>(d, hq / hkv, pairs)
                          : attn_kernel_ptr<float>(d, hq / hkv, pairs);
  int cus = device_cus();
  int cap = kern ? device_capacity(kern, 64) : 0;
  if (cap <= 0 || cus <= 0) {
    cus = 256;
    cap = 3072;
  }
  // The 16-token-tile shape: eight splits, two pairs per 16-wave workgroup,
  // when the batch fills between half the device's wave slots and two rounds.
  if (bf16 && d == 128 && hq == 8 * hkv && cap / cus == 16 && k >= 8 * 16 && pairs * 8 * 2 >= cap &&
      pairs * 8 <= 2LL * cap)
    return 8;
  if (cap / cus == 12 && k >= 6 * 32 && pairs * 6 <= cap && pairs * 6 * 2 >= cap) return 6;
  const int s = attn_default_splits(rows, hq, hkv, d, k, bf16);
  int f = 1;
  while (f * 2 <= s && f * 2 <= 8 && f * 2 <= k) f *= 2;
  return f;
}

}  // namespace dsa
