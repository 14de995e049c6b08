// Prefill group attention over the union of a group's selections
// (Megatron-LM pull request 7211, commit "--dsa-inference-backend flashinfer
// ...": prefill tiles attend each 8-token group over the union of the keys
// its tokens selected, with a per-token bitmask; commit "Restore the
// upstream Blackwell FP32 probability reduction": probabilities stay fp32
// through the value reduction).
//
// Consecutive prefill rows of one request select overlapping keys. A group of
// up to 8 such rows reads each key of the union of their selections once,
// and for one KV head its 8 rows x 8 query heads = 64 query rows make dense
// matrix tiles: the contraction is compute-bound, so it runs on the matrix
// cores (decode rows, with one row per group, stay on the vector kernel).
// Row r of the group attends only the keys it selected: the union keeps one
// mask bit per row, and a key without the row's bit scores -inf for it. The
// result is dsa_sparse_attn with one split followed by dsa_merge, up to
// rounding order.
//
// One workgroup of 4 waves per (group, KV head); wave w owns query rows
// 16w .. 16w + 15, i.e. group rows 2w and 2w + 1, all 8 heads each.
//   * union: positions are taken in windows of kWin from the smallest one
//     not yet consumed; every row's selections inside the window (a run of
//     its ascending list) set their row's bit in an LDS byte map, which is
//     then compacted in position order into (offset, mask) entries;
//   * each entry's cache row is resolved through the block table once per
//     window; tiles of 32 union keys: the 4 waves stage the keys' K rows and
//     transposed V rows for the KV head in LDS (the next tile's loads in
//     flight while this one is computed);
//   * scores: v_mfma_f32_16x16x32_bf16, query rows as A (held in registers),
//     keys as B; masked keys give -inf; online softmax per query row in
//     base 2, fp32, against a deferred reference (raised, with a rescale,
//     only when a score overtakes it by 2^8);
//   * values: the fp32 probabilities leave the accumulator layout through
//     LDS and are split exactly into three bf16 terms (p = hi + mid + lo: a
//     float's 24 significand bits are three bf16 significands), each
//     multiplied with V on the matrix cores and summed in fp32 -- the
//     products are exact, so this is the fp32 probability reduction.

#include "dsa_kernels.h"

namespace dsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGaThreads = 256;  // 4 waves
constexpr int kGaWin = 4096;     // positions per union window
constexpr int kGaTile = 32;      // union keys per tile
constexpr int kGaRows = 8;       // rows per group, at most
constexpr int kGaD = 128;        // head dim
constexpr int kGaG = 8;          // query heads per KV head
constexpr int kKst = kGaD + 8;   // K tile row stride (elements): B-fragment reads hit distinct banks
constexpr int kVst = kGaTile + 8;  // transposed V row stride (elements)
constexpr int kPst = kGaTile + 4;  // probability tile row stride (floats)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kGaSlack = 8.0f;  // log2 headroom of the deferred softmax reference

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Max / sum over the 16 lanes of a DPP row (every lane gets the result).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Orders this wave's LDS writes before its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exclusive prefix sum over the workgroup (4 waves) in thread order; sh holds
// 4 words no other code touches until the next barrier.
__device__ __forceinline__ uint32_t ga_block_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    base += i < wave ? sh[i] : 0u;
    tot += sh[i];
  }
  *total = tot;
  return base + x - v;
}

}  // namespace

__global__ __launch_bounds__(kGaThreads, 2) void group_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ groups, int hkv, int k,
    int page_shift, int max_pages, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ out_lse) {
  __shared__ uint32_t bmap[kGaWin / 4];            // the window's byte map: a row bit per position
  __shared__ uint8_t umask[kGaWin];                // union entry -> its rows' bits
  __shared__ uint32_t urow[kGaWin];                // union entry -> position, then its cache row
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kGaTile * kKst];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kGaD * kVst];   // [dim][key]
  __shared__ __attribute__((aligned(16))) float p_lds[4][16 * kPst];
  __shared__ int cursor[kGaRows];
  __shared__ int nextpos[kGaRows];
  __shared__ uint32_t scan_sh[2][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gi = (int)blockIdx.x / hkv;
  const int j = (int)blockIdx.x - gi * hkv;
  const int first = groups[2 * gi];
  const int nrows = min(max(groups[2 * gi + 1], 0), kGaRows);
  const int hq = hkv * kGaG;
  const int page_mask = (1 << page_shift) - 1;
  const int32_t* btr = bt + (size_t)row_req[first] * max_pages;
  const size_t kv_stride = (size_t)hkv * kGaD;  // elements per cache row (token)
  const uint16_t* kgroup = kc + (size_t)j * kGaD;
  const uint16_t* vgroup = vc + (size_t)j * kGaD;

  // The wave's query rows as MFMA A fragments: lane l holds query row l % 16
  // (group row 2w + (l % 16) / 8, head j * 8 + l % 8), dims kk * 32 +
  // (l / 16) * 8 .. + 8 of step kk. Rows past the group are zero.
  const int qrow = lane & 15, kgrp = lane >> 4;
  bf16x8_t qa[kGaD / 32];
  {
    const int tr = 2 * wave + (qrow >> 3);
    const int h = j * kGaG + (qrow & 7);
#pragma unroll
    for (int kk = 0; kk < kGaD / 32; ++kk) {
      if (tr < nrows)
        qa[kk] = *reinterpret_cast<const bf16x8_t*>(
            q + ((size_t)(first + tr) * hq + h) * kGaD + kk * 32 + kgrp * 8);
      else
        qa[kk] = bf16x8_t{};
    }
  }
  // Accumulator rows of this lane: (l / 16) * 4 + i, i < 4, all of group row
  // 2w + (l >= 32).
  const int my_tr = 2 * wave + (lane >> 5);
  float m[4], lsum[4];
  f32x4_t o[kGaD / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    lsum[i] = 0.0f;
  }
#pragma unroll
  for (int nt = 0; nt < kGaD / 16; ++nt) o[nt] = f32x4_t{};

  if (tid < kGaRows) cursor[tid] = 0;
  __syncthreads();

  // Staging of one tile. K: thread t takes union entry t / 8 and dims
  // (t % 8) * 16 .. + 16 (32 bytes). V: thread t takes the key pair
  // 2 (t % 16), 2 (t % 16) + 1 and dims (t / 16) * 8 .. + 8, and stores each
  // dim's two keys as one 32-bit word of the transposed tile. Entries past
  // the union re-read the tile's first key (in bounds; masked).
  const int st_key = tid >> 3, st_c = tid & 7;
  const int sv_pair = tid & 15, sv_dim = (tid >> 4) * 8;
  struct Stage {
    uint4 k[2], v[2];
  };
  auto stage_load = [&](Stage& st, int e, int n_u) {
    const int ek = e + st_key < n_u ? e + st_key : e;
    const int ev0 = e + 2 * sv_pair < n_u ? e + 2 * sv_pair : e;
    const int ev1 = e + 2 * sv_pair + 1 < n_u ? e + 2 * sv_pair + 1 : e;
    const uint4* ks = reinterpret_cast<const uint4*>(kgroup + (size_t)urow[ek] * kv_stride + st_c * 16);
    st.k[0] = ks[0];
    st.k[1] = ks[1];
    st.v[0] = *reinterpret_cast<const uint4*>(vgroup + (size_t)urow[ev0] * kv_stride + sv_dim);
    st.v[1] = *reinterpret_cast<const uint4*>(vgroup + (size_t)urow[ev1] * kv_stride + sv_dim);
  };
  auto stage_store = [&](const Stage& st) {
    uint4* kd = reinterpret_cast<uint4*>(k_lds + st_key * kKst + st_c * 16);
    kd[0] = st.k[0];
    kd[1] = st.k[1];
    const uint32_t a[4] = {st.v[0].x, st.v[0].y, st.v[0].z, st.v[0].w};
    const uint32_t b[4] = {st.v[1].x, st.v[1].y, st.v[1].z, st.v[1].w};
    uint32_t* vd = reinterpret_cast<uint32_t*>(v_lds) + sv_pair;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dims sv_dim + 2w (low halves) and sv_dim + 2w + 1 (high halves)
      vd[(sv_dim + 2 * w) * (kVst / 2)] = (a[w] & 0xFFFFu) | (b[w] << 16);
      vd[(sv_dim + 2 * w + 1) * (kVst / 2)] = (a[w] >> 16) | (b[w] & 0xFFFF0000u);
    }
  };

  const int32_t* irow_base = idx + (size_t)first * k;
  for (;;) {
    // ---- the next window: from the smallest position not yet consumed ----
    if (tid < kGaRows) {
      int c = cursor[tid];
      int p = (tid < nrows && c < k) ? irow_base[(size_t)tid * k + c] : -1;
      nextpos[tid] = p >= 0 ? p : INT32_MAX;
    }
    for (int i = tid; i < kGaWin / 4; i += kGaThreads) bmap[i] = 0u;
    __syncthreads();
    int w0 = INT32_MAX;
#pragma unroll
    for (int i = 0; i < kGaRows; ++i) w0 = min(w0, nextpos[i]);
    if (w0 == INT32_MAX) break;  // uniform: every row's selection consumed
    const int w1 = w0 > INT32_MAX - kGaWin ? INT32_MAX : w0 + kGaWin;
    // ---- each row's run inside the window sets its bit (32 threads a row) ----
    {
      const int i = tid >> 5, l32 = tid & 31;
      if (i < nrows) {
        const int32_t* ir = irow_base + (size_t)i * k;
        int c = cursor[i];
        for (;;) {
          // 128 entries per round trip; the row's list ascends, so its
          // selections inside the window are the leading in-window ones.
          int p[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int sidx = c + 32 * u + l32;
            p[u] = sidx < k ? ir[sidx] : -1;
          }
          int cnt = 0;
          bool more = true;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool in = more && p[u] >= w0 && p[u] < w1;
            const uint32_t half = (uint32_t)(__ballot(in) >> (tid & 32));
            const int run = half == 0xFFFFFFFFu ? 32 : __builtin_ctz(~half);
            if (in && l32 < run)
              atomicOr(&bmap[(p[u] - w0) >> 2], 1u << ((((p[u] - w0) & 3) << 3) + i));
            if (more) cnt += run;
            more = more && run == 32;
          }
          c += cnt;
          if (cnt < 128) break;
        }
        if (l32 == 0) cursor[i] = c;
      }
    }
    __syncthreads();
    // ---- compaction: positions with a bit, in order ----
    uint32_t n_u;
    {
      uint32_t wds[4];
      uint32_t cnt = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wds[u] = bmap[tid * 4 + u];
#pragma unroll
        for (int b = 0; b < 4; ++b) cnt += ((wds[u] >> (8 * b)) & 0xFFu) != 0u;
      }
      uint32_t o = ga_block_scan(cnt, scan_sh[0], &n_u);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t msk = (wds[u] >> (8 * b)) & 0xFFu;
          if (msk) {
            umask[o] = (uint8_t)msk;
            urow[o] = (uint32_t)(w0 + tid * 16 + u * 4 + b);
            ++o;
          }
        }
    }
    __syncthreads();
    // Every entry's cache row through the block table at once (one round
    // trip per window instead of a dependent lookup per tile).
    for (int e = tid; e < (int)n_u; e += kGaThreads) {
      const int p = (int)urow[e];
      urow[e] = ((uint32_t)btr[p >> page_shift] << page_shift) | (uint32_t)(p & page_mask);
    }
    __syncthreads();

    // ---- tiles of the window's union ----
    // The next tile's K and V loads are in flight (registers) while this
    // tile is computed; every wave reads the tile in LDS, so a barrier closes
    // each tile before the next is stored.
    const int ntiles = ((int)n_u + kGaTile - 1) / kGaTile;
    Stage st;
    stage_load(st, 0, (int)n_u);
    stage_store(st);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int e0 = t * kGaTile;
      if (t + 1 < ntiles) stage_load(st, e0 + kGaTile, (int)n_u);
      // Scores: 16 query rows x 32 keys.
      f32x4_t s[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        s[n] = f32x4_t{};
#pragma unroll
        for (int kk = 0; kk < kGaD / 32; ++kk) {
          const bf16x8_t kb = *reinterpret_cast<const bf16x8_t*>(
              k_lds + (n * 16 + qrow) * kKst + kk * 32 + kgrp * 8);
          s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], kb, s[n], 0, 0, 0);
        }
      }
      // Mask: key n * 16 + l % 16 of the tile, for group row my_tr.
      bool ok[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int e = e0 + n * 16 + qrow;
        ok[n] = e < (int)n_u && ((umask[min(e, kGaWin - 1)] >> my_tr) & 1u);
      }
      // Online softmax against a deferred reference: a row's m is raised to
      // its running max (and its sum and outputs rescaled) only when a score
      // overtakes it by more than 2^kGaSlack, so most tiles skip the
      // rescale; o and the sum share the reference, so the normalized
      // result is the same and every probability stays <= 2^kGaSlack.
      bool over = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = fmaxf(ok[0] ? s[0][i] * scale_log2 : -INFINITY,
                              ok[1] ? s[1][i] * scale_log2 : -INFINITY);
        over |= x > m[i] + kGaSlack;
      }
      if (__ballot(over) != 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = fmaxf(ok[0] ? s[0][i] * scale_log2 : -INFINITY,
                                ok[1] ? s[1][i] * scale_log2 : -INFINITY);
          const float mt = row16_max(x);
          const bool up = mt > m[i] + kGaSlack;
          // m = -inf (no selected key yet): alpha = 0 clears what is zero.
          const float alpha = up ? __builtin_amdgcn_exp2f(m[i] - mt) : 1.0f;
          lsum[i] *= alpha;
#pragma unroll
          for (int nt = 0; nt < kGaD / 16; ++nt) o[nt][i] *= alpha;
          m[i] = up ? mt : m[i];
        }
      }
      float pv[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // A masked key has probability 0 whatever the reference (before a
        // row's first selected key m is still -inf).
        pv[0][i] = ok[0] ? __builtin_amdgcn_exp2f(s[0][i] * scale_log2 - m[i]) : 0.0f;
        pv[1][i] = ok[1] ? __builtin_amdgcn_exp2f(s[1][i] * scale_log2 - m[i]) : 0.0f;
        lsum[i] += pv[0][i] + pv[1][i];
      }
      // Probabilities to the A layout through LDS (row l % 16, keys
      // (l / 16) * 8 .. + 8), split into three exact bf16 terms.
      float* pw = p_lds[wave];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[(kgrp * 4 + i) * kPst + n * 16 + qrow] = pv[n][i];
      wave_lds_sync();
      bf16x8_t ph, pm, pl;
      {
        const float4 x0 = *reinterpret_cast<const float4*>(pw + qrow * kPst + kgrp * 8);
        const float4 x1 = *reinterpret_cast<const float4*>(pw + qrow * kPst + kgrp * 8 + 4);
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint16_t hb[8], mb[8], lb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u0 = __float_as_uint(xs[e]);
          const float h = __uint_as_float(u0 & 0xFFFF0000u);
          const float r1 = xs[e] - h;  // exact
          const float mid = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
          const float r2 = r1 - mid;   // exact
          hb[e] = (uint16_t)(u0 >> 16);
          mb[e] = (uint16_t)(__float_as_uint(mid) >> 16);
          lb[e] = (uint16_t)(__float_as_uint(r2) >> 16);  // exact: at most 8 bits left
        }
        ph = __builtin_bit_cast(bf16x8_t, hb);
        pm = __builtin_bit_cast(bf16x8_t, mb);
        pl = __builtin_bit_cast(bf16x8_t, lb);
      }
      // Values: O[16 x 128] += P[16 x 32] . V[32 x 128], three terms.
#pragma unroll
      for (int nt = 0; nt < kGaD / 16; ++nt) {
        const bf16x8_t vb = *reinterpret_cast<const bf16x8_t*>(
            v_lds + (nt * 16 + qrow) * kVst + kgrp * 8);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pm, vb, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[nt], 0, 0, 0);
      }
      __syncthreads();
      if (t + 1 < ntiles) {
        stage_store(st);
        __syncthreads();
      }
    }
    // The next window rebuilds the byte map and the union list after this
    // barrier (every read of them is done).
    __syncthreads();
  }

  // ---- the rows' outputs ----
  if (my_tr < nrows) {
    const int r = first + my_tr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float l = row16_sum(lsum[i]);
      const bool any = l > 0.0f;
      const float inv = any ? 1.0f / l : 0.0f;
      const int h = j * kGaG + ((kgrp * 4 + i) & 7);
      uint16_t* orow = out + ((size_t)r * hq + h) * kGaD;
#pragma unroll
      for (int nt = 0; nt < kGaD / 16; ++nt) orow[nt * 16 + qrow] = bf16_rne(o[nt][i] * inv);
      if (out_lse && qrow == 0)
        out_lse[(size_t)r * hq + h] = any ? (m[i] + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

hipError_t launch_group_attn(const void* q, const void* kc, const void* vc, const int32_t* bt,
                             const int32_t* row_req, const int32_t* idx, const int32_t* groups,
                             int num_groups, int hkv, int k, int page_shift, int max_pages,
                             float scale, void* out, float* out_lse, hipStream_t stream) {
  hipLaunchKernelGGL(group_attn_kernel, dim3((unsigned)((long long)num_groups * hkv)),
                     dim3(kGaThreads), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), bt,
                     row_req, idx, groups, hkv, k, page_shift, max_pages, scale * kLog2e,
                     static_cast<uint16_t*>(out), out_lse);
  return hipGetLastError();
}

}  // namespace dsa
