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
// cores (decode rows, with one row per group, stay on the split attention
// kernel).
// Row r of the group attends only the keys it selected: the union keeps one
// mask bit per row, and a key without the row's bit scores -inf for it. The
// result is dsa_sparse_attn with one split followed by dsa_merge, up to
// rounding order.
//
// One workgroup of 4 waves per (group, KV head); wave w owns query rows
// 16w .. 16w + 15, i.e. group rows 2w and 2w + 1, all 8 heads each.
//   * union: positions are taken in windows of kGaWin from the smallest one
//     not yet consumed; every row's selections inside the window (a run of
//     its ascending list) set their row's bit in an LDS byte map, which is
//     then compacted in position order into (offset, mask) entries;
//   * each entry's cache row is resolved through the block table once per
//     window; tiles of 32 union keys: the keys' K and V rows for the KV head
//     are copied straight from global memory into one of two LDS buffers
//     (global_load_lds, no registers), the copies of the next tile in flight
//     while one is computed; V stays in row order and its A fragments are
//     read with the transposing ds_read_b64_tr_b16;
//   * 39 KB of LDS (windows of 1024 positions, two tile buffers) and at most
//     128 VGPRs a lane let four workgroups share a compute unit, which hides
//     more of each wave's barrier and load waits than a deeper copy
//     pipeline (three buffers, two workgroups) did;
//   * scores, transposed: S^T = K . Q^T on v_mfma_f32_16x16x32_bf16, keys as
//     A, the query rows (held in registers) as B, so each lane holds one
//     query row and eight of the tile's keys; masked keys give -inf; online
//     softmax per query row in base 2, fp32, against a deferred reference
//     (raised, with a rescale, only when a score overtakes it by 2^8);
//   * values, transposed: O^T += V^T . P^T, whose B operand is exactly what
//     the scores left in each lane (the eight keys in the order the V^T
//     fragments are read), so the probabilities never leave registers; each
//     is split exactly into three bf16 terms (p = hi + mid + lo: a float's 24
//     significand bits are three bf16 significands), each multiplied with V
//     on the matrix cores and summed in fp32 -- the products are exact, so
//     this is the fp32 probability reduction.

#include "dsa_kernels.h"

namespace dsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGaThreads = 256;  // 4 waves
constexpr int kGaWin = 1024;     // positions per union window
constexpr int kWpt = kGaWin / 4 / kGaThreads;  // byte-map words per thread in the compaction
static_assert(kWpt >= 1 && kWpt * 4 * kGaThreads == kGaWin, "the compaction covers the window exactly");
constexpr int kGaTile = 32;      // union keys per tile
constexpr int kGaRows = 8;       // rows per group, at most
constexpr int kGaD = 128;        // head dim
constexpr int kGaG = 8;          // query heads per KV head
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait until at most 4 or 0 vector memory instructions
// are outstanding, nothing else.
constexpr int kWaitVm4 = 4 | (7 << 4) | (15 << 8);
constexpr int kWaitVm0 = 0 | (7 << 4) | (15 << 8);
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);  // LDS / scalar only
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kGaSlack = 8.0f;  // log2 headroom of the deferred softmax reference

// Max / sum over the four lanes l % 16 + 16 g, g < 4 (the lanes holding one
// query row), every one of them getting the result: two row swaps.
__device__ __forceinline__ float groups4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float groups4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Tile rows are stored unpadded (256 bytes per key) with the 16 16-byte
// pieces of key j's row permuted: piece p sits in slot p ^ f(j). For K,
// f(j) = j % 16 spreads the 16 keys of an A-fragment read over all banks; for
// V (read with the transposing ds_read_b64_tr_b16: one instruction covers 16
// consecutive keys, two pieces each) f(j) = 2 (j % 8) puts those 32 pieces
// two to a slot, the fewest a 512-byte read allows.
__device__ __forceinline__ int k_slot_xor(int j) { return j & 15; }
__device__ __forceinline__ int v_slot_xor(int j) { return (j & 7) << 1; }

typedef __attribute__((address_space(1))) void ga_gvoid;
typedef __attribute__((address_space(3))) void ga_lvoid;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t ga_lds_bf16x4;

// A workgroup barrier without the memory fences of __syncthreads, whose
// release would wait for every load in flight (the next tiles' copies
// included). LDS reads and writes on either side stay on their side (the
// empty asm for the compiler, the scheduling barriers for the backend); the
// caller waits for whatever the other waves must see.
__device__ __forceinline__ void ga_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
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

// Four workgroups per compute unit: at most 128 VGPRs a lane.
__global__ __launch_bounds__(kGaThreads, 4) void group_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ groups, int hkv, int k,
    int page_shift, int max_pages, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ out_lse) {
  __shared__ uint32_t bmap[kGaWin / 4];            // the window's byte map: a row bit per position
  __shared__ __attribute__((aligned(4))) uint8_t umask[kGaWin];  // union entry -> its rows' bits
  __shared__ uint32_t urow[kGaWin];                // union entry -> position, then its cache row
  // Tile buffers (K and V of two tiles): [key][128 dims], pieces permuted
  // per key. Separate arrays, each named where it is used, so that the
  // compiler can tell a tile's reads from the copies into the other buffer
  // and waits only for the copies it reads.
  __shared__ __attribute__((aligned(16))) uint16_t kbuf0[kGaTile * kGaD], vbuf0[kGaTile * kGaD];
  __shared__ __attribute__((aligned(16))) uint16_t kbuf1[kGaTile * kGaD], vbuf1[kGaTile * kGaD];
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

  // The wave's query rows as MFMA B fragments: lane l holds query row l % 16
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
  // This lane's query row (its scores, reference, running sum and the
  // column of O^T it accumulates: dims nt * 16 + (l / 16) * 4 + i).
  const int my_tr = 2 * wave + (qrow >> 3);
  float m = -INFINITY, lsum = 0.0f;
  f32x4_t o[kGaD / 16];
#pragma unroll
  for (int nt = 0; nt < kGaD / 16; ++nt) o[nt] = f32x4_t{};

  if (tid < kGaRows) cursor[tid] = 0;
  __syncthreads();

  // A tile's K and V rows go straight from global memory to LDS (no
  // registers): each of a wave's four load instructions covers four keys'
  // 256-byte rows, lane l taking piece (l % 16) ^ f(key) of key l / 16, so a
  // lane's 16 bytes land in slot l % 16. Entries past the union re-read the
  // tile's first key (in bounds; masked).
  auto issue_tile = [&](int t, uint16_t* kdst, uint16_t* vdst, int n_u) {
    const int e0 = t * kGaTile;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * wave + u;           // keys 4i .. 4i + 3 of the tile
      const int kk = 4 * i + (lane >> 4);
      const int sl = lane & 15;
      const int e = e0 + kk < n_u ? e0 + kk : e0;
      const size_t row = urow[e];
      const uint16_t* kp = kgroup + row * kv_stride + 8 * (sl ^ k_slot_xor(kk));
      const uint16_t* vp = vgroup + row * kv_stride + 8 * (sl ^ v_slot_xor(kk));
      __builtin_amdgcn_global_load_lds((ga_gvoid*)kp, (ga_lvoid*)(kdst + i * 4 * kGaD), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((ga_gvoid*)vp, (ga_lvoid*)(vdst + i * 4 * kGaD), 16, 0, 0);
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
    // Thread t owns the kWpt map words from t * kWpt (4 positions a word).
    uint32_t n_u;
    {
      uint32_t wds[kWpt];
      uint32_t cnt = 0;
#pragma unroll
      for (int u = 0; u < kWpt; ++u) {
        wds[u] = bmap[tid * kWpt + u];
#pragma unroll
        for (int b = 0; b < 4; ++b) cnt += ((wds[u] >> (8 * b)) & 0xFFu) != 0u;
      }
      uint32_t o = ga_block_scan(cnt, scan_sh[0], &n_u);
#pragma unroll
      for (int u = 0; u < kWpt; ++u)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t msk = (wds[u] >> (8 * b)) & 0xFFu;
          if (msk) {
            umask[o] = (uint8_t)msk;
            urow[o] = (uint32_t)(w0 + tid * 4 * kWpt + u * 4 + b);
            ++o;
          }
        }
    }
    __syncthreads();
    // Every entry's cache row through the block table at once (one round
    // trip per window instead of a dependent lookup per tile); the mask
    // bytes past the union up to the last tile's end are cleared, so those
    // slots select no row.
    for (int e = tid; e < (int)n_u; e += kGaThreads) {
      const int p = (int)urow[e];
      urow[e] = ((uint32_t)btr[p >> page_shift] << page_shift) | (uint32_t)(p & page_mask);
    }
    for (int e = (int)n_u + tid; e < (((int)n_u + kGaTile - 1) & ~(kGaTile - 1)); e += kGaThreads)
      umask[e] = 0u;
    __syncthreads();

    // ---- tiles of the window's union ----
    // Tile t is computed from buffer t % 2 while the copies of tile t + 1
    // are in flight; a wave's own copies of tile t are complete when at most
    // the next tile's four instructions are outstanding, and a barrier then
    // covers every wave's. A second barrier closes each tile before its
    // buffer is loaded again.
    const int ntiles = ((int)n_u + kGaTile - 1) / kGaTile;
    // One tile: start the next tile's copies, wait for this one's, compute
    // it from (k_lds, v_lds), then close it before its buffers are reused.
    auto tile = [&](int t, const uint16_t* k_lds, const uint16_t* v_lds, auto&& issue_ahead) {
      const int e0 = t * kGaTile;
      if (t + 1 < ntiles) {
        issue_ahead();
        __builtin_amdgcn_s_waitcnt(kWaitVm4);
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      }
      ga_barrier();  // every wave's copies of tile t are in LDS
      // Scores S^T: keys n * 16 + 4 (l / 16) + i of the tile (i < 4) for
      // query row l % 16.
      f32x4_t s[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        s[n] = f32x4_t{};
#pragma unroll
        for (int kk = 0; kk < kGaD / 32; ++kk) {
          const int key = n * 16 + qrow;
          const bf16x8_t kb = *reinterpret_cast<const bf16x8_t*>(
              k_lds + key * kGaD + 8 * ((kk * 4 + kgrp) ^ k_slot_xor(key)));
          s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qa[kk], s[n], 0, 0, 0);
        }
      }
      // Mask: the four union entries e0 + n * 16 + 4 (l / 16) .. + 3 in one
      // word of the byte map, bit my_tr of each (slots past the union hold
      // no bits); a masked key scores -inf.
      bool ok[2][4];
      float sv[2][4];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const uint32_t mw = *reinterpret_cast<const uint32_t*>(umask + e0 + n * 16 + 4 * kgrp) >> my_tr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ok[n][i] = (mw >> (8 * i)) & 1u;
          sv[n][i] = ok[n][i] ? s[n][i] : -INFINITY;
        }
      }
      // Online softmax in base 2 (x = s * scale_log2) against a deferred
      // reference: a row's m is raised to its running max (and its sum and
      // outputs rescaled) only when a score overtakes it by more than
      // 2^kGaSlack, so most tiles skip the rescale; o and the sum share the
      // reference, so the normalized result is the same and every
      // probability stays <= 2^kGaSlack. The lane's largest x is its largest
      // s times the (positive) scale: rounding keeps the order.
      float xm = fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3]));
      xm = fmaxf(xm, fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3]))) * scale_log2;
      if (__ballot(xm > m + kGaSlack) != 0) {
        const float mt = groups4_max(xm);
        const bool up = mt > m + kGaSlack;
        // m = -inf (no selected key yet): alpha = 0 clears what is zero.
        const float alpha = up ? __builtin_amdgcn_exp2f(m - mt) : 1.0f;
        lsum *= alpha;
#pragma unroll
        for (int nt = 0; nt < kGaD / 16; ++nt) o[nt] *= alpha;
        m = up ? mt : m;
      }
      // Probabilities (a masked key has 0 whatever the reference: before a
      // row's first selected key m is still -inf), split into three exact
      // bf16 terms: the B operands of O^T += V^T . P^T, k index 8 (l / 16) +
      // 4 n + i holding key n * 16 + 4 (l / 16) + i.
      uint16_t hb[8], mb[8], lb[8];
      float ps = 0.0f;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = ok[n][i] ? __builtin_amdgcn_exp2f(fmaf(s[n][i], scale_log2, -m)) : 0.0f;
          ps += p;
          const uint32_t u0 = __float_as_uint(p);
          const float r1 = p - __uint_as_float(u0 & 0xFFFF0000u);  // exact
          const uint32_t u1 = __float_as_uint(r1);
          const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);  // exact, <= 8 bits left
          hb[4 * n + i] = (uint16_t)(u0 >> 16);
          mb[4 * n + i] = (uint16_t)(u1 >> 16);
          lb[4 * n + i] = (uint16_t)(__float_as_uint(r2) >> 16);
        }
      lsum += ps;
      const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, hb);
      const bf16x8_t pm = __builtin_bit_cast(bf16x8_t, mb);
      const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, lb);
      // Values: O^T[128 x 16] += V^T[128 x 32] . P^T[32 x 16], three terms.
      // The A fragment (dim nt * 16 + l % 16, the eight keys of this lane's
      // probabilities) comes from two transposing reads: lane j of a 16-lane
      // group addresses the four dims nt * 16 + 4 (j % 4) .. + 4 of key
      // hh * 16 + 4 (l / 16) + j / 4, and lane m receives dim nt * 16 + m of
      // those four keys.
      const int jq = qrow & 3, jk = qrow >> 2;
#pragma unroll
      for (int nt = 0; nt < kGaD / 16; ++nt) {
        bf16x4_t vh[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int key = hh * 16 + kgrp * 4 + jk;
          const int d = nt * 16 + 4 * jq;
          const uint16_t* src = v_lds + key * kGaD + 8 * ((d >> 3) ^ v_slot_xor(key)) + (d & 7);
          vh[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (ga_lds_bf16x4*)(__attribute__((address_space(3))) uint16_t*)src);
        }
        const bf16x8_t vb = {vh[0][0], vh[0][1], vh[0][2], vh[0][3],
                             vh[1][0], vh[1][1], vh[1][2], vh[1][3]};
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, ph, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pm, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pl, o[nt], 0, 0, 0);
      }
      // Every wave's reads of this tile's buffers are done (their MFMAs have
      // issued) before any wave copies a later tile into them.
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      ga_barrier();
    };
    issue_tile(0, kbuf0, vbuf0, (int)n_u);
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, kbuf0, vbuf0, [&] { issue_tile(t + 1, kbuf1, vbuf1, (int)n_u); });
      if (t + 1 >= ntiles) break;
      tile(t + 1, kbuf1, vbuf1, [&] { issue_tile(t + 2, kbuf0, vbuf0, (int)n_u); });
    }
    // The next window rebuilds the byte map and the union list after this
    // barrier (every read of them is done).
    __syncthreads();
  }

  // ---- the rows' outputs ----
  // The row's sum over the four lanes holding it (every one of them joins).
  const float l = groups4_sum(lsum);
  if (my_tr < nrows) {
    const int r = first + my_tr;
    const bool any = l > 0.0f;
    const float inv = any ? 1.0f / l : 0.0f;
    const int h = j * kGaG + (qrow & 7);
    uint16_t* orow = out + ((size_t)r * hq + h) * kGaD + 4 * kgrp;
#pragma unroll
    for (int nt = 0; nt < kGaD / 16; ++nt) {
      const uint32_t lo = bf16_rne(o[nt][0] * inv) | ((uint32_t)bf16_rne(o[nt][1] * inv) << 16);
      const uint32_t hi = bf16_rne(o[nt][2] * inv) | ((uint32_t)bf16_rne(o[nt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + nt * 16) = make_uint2(lo, hi);
    }
    if (out_lse && kgrp == 0)
      out_lse[(size_t)r * hq + h] = any ? (m + __log2f(l)) * kLn2 : -INFINITY;
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
