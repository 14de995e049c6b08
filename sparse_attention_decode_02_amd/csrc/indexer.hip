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
// Work: a workgroup takes (score block, key chunk). Chunks past a row's
// length exit at once, so the launch depends only on (blocks, width) while
// the work follows the real lengths. On the bf16 path, blocks of one row
// (decode) go to the row kernel described above, whose waves stream keys
// through registers; blocks of several rows of one request (prefill) go to
// the block kernel, whose
// workgroup stages each key tile once in LDS for all its rows, so a chunk's
// keys cross HBM/L2 once per block rather than once per row and the
// contraction runs on the matrix cores at prefill's arithmetic intensity.

#include "radix_select.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // a native vector (promotes to registers)

constexpr int kIdxThreads = 256;  // 4 waves
constexpr int kTileKeys = 16;     // keys per MFMA tile (N of 16x16x32)
constexpr int kKeyBufs = 3;       // key tiles per wave: 2 in flight + 1 on the matrix cores
constexpr int kMaxChunkKeys = 2048;  // keys per workgroup chunk, at most (scores staged in LDS)

// Workgroup -> item: items in groups of G are dealt round-robin to the 8
// XCDs (workgroup i runs on XCD i % 8), so the items of a group share their
// XCD's L2 while work that clusters in one range of items (short causal rows
// in the low chunks, a few long rows at the end of the batch) still spreads
// over every XCD. The grid is padded to a multiple of 8 * G; items past the
// end exit.
template <int G>
__device__ __forceinline__ int xcd_grouped(int wg) {
  const int x = wg & 7, j = wg >> 3;
  return ((j / G) * 8 + x) * G + j % G;
}

inline int xcd_grouped_grid(int total, int G) { return (total + 8 * G - 1) / (8 * G) * (8 * G); }

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
template <int HT, int DI, bool BAL = false>
__global__ __launch_bounds__(kIdxThreads, 4) void indexer_mfma_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w,
    const uint16_t* __restrict__ kc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ row_req, const int32_t* __restrict__ row_len,
    const int32_t* __restrict__ blocks, float* __restrict__ scores, int width, int page_shift,
    int max_pages, int chunk_keys, int chunks, int total, int score_row0, int single_only,
    uint32_t* __restrict__ hist) {
  constexpr int H = HT * 16;
  constexpr int KS = DI / 32;  // MFMA steps per head tile
  constexpr int QST = DI + 8;  // padded LDS row (elements): the 16 rows read together hit distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[H * QST];
  // The chunk's score histogram (with `hist`): two 16-bit counters per word
  // (a chunk holds at most 2048 keys), bins 2i and 2i + 1 in word i.
  __shared__ uint32_t h_lds[kHistBins / 2];
  __shared__ __attribute__((aligned(16))) float w_lds[H];
  __shared__ __attribute__((aligned(16))) float s_lds[kMaxChunkKeys];  // the chunk's scores
  __shared__ uint32_t bal_sh[kIdxThreads / 64];
  __shared__ int bal_item;

  const int tid = threadIdx.x;
  // Items are (block, chunk) pairs. Beside the block kernel only some blocks
  // are this kernel's, so its items are dealt round-robin over the XCDs;
  // alone, consecutive items (the chunks of a row) share an XCD, each XCD
  // taking an equal range of (block, chunk) slots. A batch of ragged one-row
  // blocks (BAL: at most one block per thread) would load the XCDs
  // unevenly that way (a range holds whole rows), so there the active items
  // -- chunks that start inside their row -- are numbered in row order,
  // each XCD takes an equal contiguous share of them (workgroup i runs on
  // XCD i % 8), and workgroup j of an XCD's J takes items j, j + J, ... of
  // its share: any grid covers every item.
  int kbeg, kend, kstep = 1;
  uint32_t bal_pre = 0, bal_cnt = 0;  // BAL: thread t's block's first item and count
  if constexpr (BAL) {
    const int nb = total / chunks;
    if (tid < nb) {
      const int L = row_len[blocks ? blocks[2 * tid] : tid];
      bal_cnt = L > 0 ? (uint32_t)min((L + chunk_keys - 1) / chunk_keys, chunks) : 0u;
    }
    uint32_t na;
    bal_pre = block_exclusive_scan<kIdxThreads / 64>(bal_cnt, bal_sh, &na);
    const int n = (int)na, x = (int)(blockIdx.x & 7), q = n >> 3, rem = n & 7;
    const int start = x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q;
    kbeg = start + (int)(blockIdx.x >> 3);
    kend = start + (x < rem ? q + 1 : q);
    kstep = (int)(gridDim.x >> 3);
  } else {
    kbeg = single_only ? xcd_grouped<2>(blockIdx.x) : xcd_contiguous(blockIdx.x, total);
    kend = min(kbeg + 1, total);
  }
  for (int k = kbeg; k < kend; k += kstep) {
    int item = k;
    if constexpr (BAL) {
      __syncthreads();  // every thread has read the previous item
      if (bal_cnt > 0u && bal_pre <= (uint32_t)k && (uint32_t)k < bal_pre + bal_cnt)
        bal_item = (int)tid * chunks + (k - (int)bal_pre);
      __syncthreads();
      item = bal_item;
    }
    const int b = item / chunks;
    const int chunk0 = (item - b * chunks) * chunk_keys;
    int first = b, nrows = 1;
    if (blocks) {
      first = blocks[2 * b];
      nrows = blocks[2 * b + 1];
      if (single_only && nrows > 1) continue;  // the block kernel's
    }
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
        if (hist)
          for (int i = tid; i < kHistBins / 2; i += kIdxThreads) h_lds[i] = 0u;
      }
      __syncthreads();

      float4 wr[HT];
  #pragma unroll
      for (int t = 0; t < HT; ++t)
        wr[t] = *reinterpret_cast<const float4*>(&w_lds[t * 16 + grp * 4]);
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
            const bf16x8 qv =
                *reinterpret_cast<const bf16x8*>(&q_lds[t * 16 * QST + kk * 32 + qoff]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv, kf[kk], acc, 0, 0, 0);
          }
          part = fmaf(wr[t].x, relu(acc[0]), part);
          part = fmaf(wr[t].y, relu(acc[1]), part);
          part = fmaf(wr[t].z, relu(acc[2]), part);
          part = fmaf(wr[t].w, relu(acc[3]), part);
        }
        part = sum_rows(part) + 0.0f;
        const int s = base + kl;
        if (grp == 0 && s < L) {
          s_lds[s - chunk0] = part;
          if (hist) {
            // Counted as it is made, under the key loads in flight.
            const uint32_t bin = order_key(part) >> kHistShift;
            atomicAdd(&h_lds[bin >> 1], 1u << ((bin & 1u) << 4));
          }
        }
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
      if (hist) {
        // The chunk's counts (the selection's threshold histogram: scores by
        // the top 12 bits of their order keys) join the row's: one global
        // atomic per non-empty bin. The next row clears h_lds only after a
        // barrier.
        uint32_t* hr = hist + (size_t)(r - score_row0) * kHistBins;
        for (int i = tid; i < kHistBins / 2; i += kIdxThreads) {
          const uint32_t n = h_lds[i];
          if (n & 0xFFFFu) atomicAdd(&hr[2 * i], n & 0xFFFFu);
          if (n >> 16) atomicAdd(&hr[2 * i + 1], n >> 16);
        }
      }
    }
  }
}

// Score blocks of several rows (prefill): the roles of the row kernel are
// swapped so that a chunk's keys cross HBM/L2 once per block instead of once
// per row. Wave w of the 8-wave workgroup holds one row's query block in
// registers as MFMA A fragments (HT*KS fragments of 8 bf16); the workgroup
// stages the chunk's keys 128 at a time in LDS (rows padded to DI + 8
// elements, so the 16 keys of a B fragment read hit distinct banks) and every
// row of the block reads its B fragments there. Each wave scores its row's
// tiles in the same MFMA order and with the same fp32 epilogue as the row
// kernel, so the scores are the same bits. The rows of a block share a
// request (the block plan's contract), so one block-table row serves all of
// them; its entries for the chunk are read once into LDS.
//
// Blocks of 2 <= R < 8 rows give each row 8 / R waves, which split the
// stage's tiles; blocks of more than 8 rows are scored 8 rows at a time.
// Blocks of one row are left to the row kernel, launched beside this one.
constexpr int kBlkThreads = 512;                       // 8 waves
constexpr int kBlkWaves = kBlkThreads / 64;
constexpr int kStageKeys = 128;                        // keys per LDS stage (8 tiles)
constexpr int kStageTiles = kStageKeys / kTileKeys;
constexpr int kMaxBlkChunk = 8192;                     // keys per workgroup chunk, at most
constexpr int kMinBlkChunk = 512;
constexpr int kBlkGroup = 8;  // consecutive (chunk, block) items an XCD takes together

// One LDS stage of the block kernel: thread t holds pieces (key0 + i * KSTEP,
// c0) for i < SV, with key0 = t / CPK and c0 = t % CPK (CPK 16-byte pieces
// per key row). Positions past `end` re-read the key at end - 1. The page of
// a position comes from pg_lds (the chunk's block-table entries from page p0).
template <int DI, int SV>
__device__ __forceinline__ void blk_fetch(u32x4 (&pre)[SV], const uint16_t* __restrict__ kc,
                                          const int* pg_lds, int s0, int end, int key0, int c0,
                                          int page_shift, int p0) {
  constexpr int KSTEP = kBlkThreads / (DI / 8);
  const int page_mask = (1 << page_shift) - 1;
#pragma unroll
  for (int i = 0; i < SV; ++i) {
    const int s = min(s0 + key0 + i * KSTEP, end - 1);
    const int page = pg_lds[(s >> page_shift) - p0];
    const size_t krow = ((size_t)page << page_shift) | (size_t)(s & page_mask);
    pre[i] = *reinterpret_cast<const u32x4*>(kc + krow * DI + c0 * 8);
  }
}

template <int DI, int SV>
__device__ __forceinline__ void blk_stash(const u32x4 (&pre)[SV], uint16_t* buf, int key0, int c0) {
  constexpr int KSTEP = kBlkThreads / (DI / 8);
  constexpr int KST = DI + 8;
  uint16_t* dst = buf + key0 * KST + c0 * 8;
#pragma unroll
  for (int i = 0; i < SV; ++i) *reinterpret_cast<u32x4*>(dst + i * KSTEP * KST) = pre[i];
}

template <int HT, int DI>
__global__ __launch_bounds__(kBlkThreads, 4) void indexer_block_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w,
    const uint16_t* __restrict__ kc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ row_req, const int32_t* __restrict__ row_len,
    const int32_t* __restrict__ blocks, float* __restrict__ scores, int width, int page_shift,
    int max_pages, int chunk_keys, int num_blocks, int total, int score_row0) {
  constexpr int H = HT * 16;
  constexpr int KS = DI / 32;
  constexpr int KST = DI + 8;                          // padded LDS key row (elements)
  constexpr int CPK = DI / 8;                          // 16-byte pieces of a key row
  constexpr int SV = kStageKeys * CPK / kBlkThreads;   // pieces per thread per stage
  static_assert(SV * kBlkThreads == kStageKeys * CPK, "stage must split evenly over the threads");
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kStageKeys * KST];
  __shared__ int pg_lds[kMaxBlkChunk / 16 + 1];
  __shared__ __attribute__((aligned(16))) float w_lds[kBlkWaves][H];  // each wave's row weights

  // Chunk-major order, so that the blocks of a group share a chunk.
  const int item = xcd_grouped<kBlkGroup>(blockIdx.x);
  if (item >= total) return;
  const int ci = item / num_blocks;
  const int b = item - ci * num_blocks;
  const int chunk0 = ci * chunk_keys;
  const int first = blocks[2 * b], nrows = blocks[2 * b + 1];
  if (nrows < 2) return;  // the row kernel's
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const int kl = lane & 15, grp = lane >> 4;
  const int32_t* btr = bt + (size_t)row_req[first] * max_pages;
  const int key0 = tid / CPK, c0 = tid - key0 * CPK;  // this thread's first stage piece

  for (int g0 = 0; g0 < nrows; g0 += kBlkWaves) {
    const int R = min(nrows - g0, kBlkWaves);
    int lmax = 0;
    for (int i = 0; i < R; ++i) lmax = max(lmax, row_len[first + g0 + i]);
    if (chunk0 >= lmax) continue;  // uniform over the workgroup
    const int end = min(lmax, chunk0 + chunk_keys);
    const int P = kBlkWaves / R;  // waves per row
    const int sub = wv / R;
    const bool active = sub < P;
    const int r = first + g0 + (wv - sub * R);
    const int L = active ? row_len[r] : 0;
    float* out = scores + (size_t)(r - score_row0) * width;

    const int p0 = chunk0 >> page_shift;
    const int np = ((end - 1) >> page_shift) - p0 + 1;
    __syncthreads();  // the previous group is done with pg_lds and k_lds
    for (int i = tid; i < np; i += kBlkThreads) pg_lds[i] = btr[p0 + i];

    // The head weights stay in LDS (read per tile) to leave registers for
    // two workgroups per compute unit.
    bf16x8 qf[HT][KS];
    if (active) {
      const uint16_t* qrow = qI + (size_t)r * H * DI + kl * DI + grp * 8;
#pragma unroll
      for (int t = 0; t < HT; ++t) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          qf[t][kk] = *reinterpret_cast<const bf16x8*>(qrow + t * 16 * DI + kk * 32);
      }
      if (lane < H) w_lds[wv][lane] = w[(size_t)r * H + lane];
    }
    __syncthreads();  // pg_lds and w_lds are filled

    // Stage loads: CPK consecutive threads read one key's row; positions past
    // the group's end re-read its last key (valid, never stored).
    u32x4 pre[SV];
    const int nst = (end - chunk0 + kStageKeys - 1) / kStageKeys;
    const int rot = b % nst;
    auto stage = [&](int i) { return i + rot < nst ? i + rot : i + rot - nst; };
    blk_fetch<DI, SV>(pre, kc, pg_lds, chunk0 + stage(0) * kStageKeys, end, key0, c0, page_shift, p0);
    blk_stash<DI, SV>(pre, k_lds[0], key0, c0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      if (st + 1 < nst)
        blk_fetch<DI, SV>(pre, kc, pg_lds, chunk0 + stage(st + 1) * kStageKeys, end, key0, c0,
                          page_shift, p0);
      if (active) {
        const uint16_t* kb = &k_lds[st & 1][kl * KST + grp * 8];
        const int s0 = chunk0 + stage(st) * kStageKeys;
        for (int tt = sub; tt < kStageTiles; tt += P) {
          const int base = s0 + tt * kTileKeys;
          if (base >= L) break;  // wave-uniform; tiles ascend within a stage
          f32x4 acc[HT];
#pragma unroll
          for (int t = 0; t < HT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          // Waves issuing MFMAs go first, so the matrix cores stay fed while
          // other waves run their epilogues and stage copies (~4%).
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + tt * kTileKeys * KST + kk * 32);
#pragma unroll
            for (int t = 0; t < HT; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[t][kk], kf, acc[t], 0, 0, 0);
          }
          __builtin_amdgcn_s_setprio(0);
          float part = 0.0f;
#pragma unroll
          for (int t = 0; t < HT; ++t) {
            const float4 wr = *reinterpret_cast<const float4*>(&w_lds[wv][t * 16 + grp * 4]);
            part = fmaf(wr.x, relu(acc[t][0]), part);
            part = fmaf(wr.y, relu(acc[t][1]), part);
            part = fmaf(wr.z, relu(acc[t][2]), part);
            part = fmaf(wr.w, relu(acc[t][3]), part);
          }
          part = sum_rows(part);
          const int s = base + kl;
          if (grp == 0 && s < L) out[s] = part + 0.0f;
        }
      }
      if (st + 1 < nst) blk_stash<DI, SV>(pre, k_lds[(st + 1) & 1], key0, c0);
      __syncthreads();
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

static const void* indexer_block_kernel_ptr(int num_heads, int head_dim) {
  if (num_heads == 64 && head_dim == 128) return (const void*)indexer_block_kernel<4, 128>;
  if (num_heads == 32 && head_dim == 128) return (const void*)indexer_block_kernel<2, 128>;
  if (num_heads == 64 && head_dim == 64) return (const void*)indexer_block_kernel<4, 64>;
  if (num_heads == 32 && head_dim == 64) return (const void*)indexer_block_kernel<2, 64>;
  return nullptr;
}

bool indexer_uses_blocks(int rows, int num_blocks) {
  // Some block holds more than one row (the row counts are on the device).
  return num_blocks > 0 && rows > num_blocks;
}

int indexer_block_chunk_keys(int num_blocks, int width, int num_heads, int head_dim, bool full) {
  // As for the row kernel: about one round of workgroups over the device,
  // in whole stages; 2048 keys at most unless the rows fill the width (causal
  // prefill blocks of unequal length then balance over more chunks).
  const void* kern = indexer_block_kernel_ptr(num_heads, head_dim);
  int cap = kern ? device_capacity(kern, kBlkThreads) : 0;
  if (cap <= 0) cap = 256;
  const int per_block = max(1, cap / max(1, num_blocks));
  int chunk = (width + per_block - 1) / per_block;
  chunk = ((chunk + kStageKeys - 1) / kStageKeys) * kStageKeys;
  return max(kMinBlkChunk, min(full ? kMaxBlkChunk : 2048, chunk));
}

hipError_t launch_indexer_bf16(const void* q_idx, const float* w, const void* kcache,
                               const int32_t* bt, const int32_t* row_req, const int32_t* row_len,
                               const int32_t* blocks, int num_blocks, int rows, float* scores,
                               int width, int num_heads, int head_dim, int page_shift,
                               int max_pages, bool full, int score_row0, hipStream_t stream,
                               uint32_t* hist, long long total_keys) {
  const auto* q = static_cast<const uint16_t*>(q_idx);
  const auto* k = static_cast<const uint16_t*>(kcache);
  const bool with_block_kernel = blocks && indexer_uses_blocks(rows, num_blocks);
  // Beside the block kernel (matrix-core bound) the row kernel (HBM bound)
  // runs on a second stream, so the two share the compute units.
  SideStream* side = with_block_kernel ? side_stream() : nullptr;
  if (with_block_kernel && !side) return hipErrorOutOfMemory;
  std::unique_lock<std::mutex> side_lock;
  if (side) side_lock = std::unique_lock<std::mutex>(*side->lock);
  hipStream_t row_stream = stream;
  if (side) {
    hipError_t e = hipEventRecord(side->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
    if (e != hipSuccess) return e;
    row_stream = side->stream;
  }
  {
    const int single_only = with_block_kernel ? 1 : 0;
    const int chunk = indexer_chunk_keys(num_blocks, width, num_heads, head_dim, full);
    const int chunks = (width + chunk - 1) / chunk;
    const int total = num_blocks * chunks;
    int grid = single_only ? xcd_grouped_grid(total, 2) : total;
    // Ragged batches of one-row blocks balance their active items over the
    // XCDs; the row plan's key count sizes the grid (one item a workgroup
    // when it is right: each row has at most one partial chunk), and the
    // workgroups loop over their share if it is not.
    const bool balanced =
        !with_block_kernel && !full && total_keys > 0 && num_blocks == rows && rows <= kIdxThreads;
    if (balanced) {
      const long long bound = std::min<long long>(total, total_keys / chunk + num_blocks);
      grid = (int)((bound + 7) / 8 * 8);
    }
#define DSA_IDX_LAUNCH(HT, DI)                                                                 \
  do {                                                                                         \
    if (balanced)                                                                              \
      hipLaunchKernelGGL((indexer_mfma_kernel<HT, DI, true>), dim3(grid), dim3(kIdxThreads), 0, \
                         row_stream, q, w, k, bt, row_req, row_len, blocks, scores, width,     \
                         page_shift, max_pages, chunk, chunks, total, score_row0, single_only, \
                         with_block_kernel ? nullptr : hist);                                  \
    else                                                                                       \
      hipLaunchKernelGGL((indexer_mfma_kernel<HT, DI>), dim3(grid), dim3(kIdxThreads), 0,      \
                         row_stream, q, w, k, bt, row_req, row_len, blocks, scores, width,     \
                         page_shift, max_pages, chunk, chunks, total, score_row0, single_only, \
                         with_block_kernel ? nullptr : hist);                                  \
  } while (0)
    if (num_heads == 64 && head_dim == 128) DSA_IDX_LAUNCH(4, 128);
    else if (num_heads == 32 && head_dim == 128) DSA_IDX_LAUNCH(2, 128);
    else if (num_heads == 64 && head_dim == 64) DSA_IDX_LAUNCH(4, 64);
    else if (num_heads == 32 && head_dim == 64) DSA_IDX_LAUNCH(2, 64);
    else return hipErrorInvalidValue;
#undef DSA_IDX_LAUNCH
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && side) e = hipEventRecord(side->join, side->stream);
    if (e != hipSuccess) return e;
  }
  if (with_block_kernel) {
    const int chunk = indexer_block_chunk_keys(num_blocks, width, num_heads, head_dim, full);
    const int total = num_blocks * ((width + chunk - 1) / chunk);
    const int grid = xcd_grouped_grid(total, kBlkGroup);
#define DSA_IDX_BLK(HT, DI)                                                                    \
  hipLaunchKernelGGL((indexer_block_kernel<HT, DI>), dim3(grid), dim3(kBlkThreads), 0, stream,  \
                     q, w, k, bt, row_req, row_len, blocks, scores, width, page_shift,          \
                     max_pages, chunk, num_blocks, total, score_row0)
    if (num_heads == 64 && head_dim == 128) DSA_IDX_BLK(4, 128);
    else if (num_heads == 32 && head_dim == 128) DSA_IDX_BLK(2, 128);
    else if (num_heads == 64 && head_dim == 64) DSA_IDX_BLK(4, 64);
    else if (num_heads == 32 && head_dim == 64) DSA_IDX_BLK(2, 64);
    else return hipErrorInvalidValue;
#undef DSA_IDX_BLK
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, side->join, 0);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipSuccess;
  // Rows scored by the block kernel are counted from their written scores.
  if (hist && with_block_kernel)
    e = launch_score_hist(scores, row_len, rows, width, hist, false, stream);
  return e;
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
