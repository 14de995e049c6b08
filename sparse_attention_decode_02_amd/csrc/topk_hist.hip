// Length-bounded exact top-k from a histogram of each row's scores
// (Megatron-LM pull request 7211: commit "When a step's context bound
// reaches 64K keys, each row now thresholds at a sampled score ...": a
// threshold per row, a filter that keeps the keys reaching it, and the exact
// top k taken among those candidates; commit "Replace the CuTe decode
// kernels with two Triton kernels": a row is read only up to its length).
//
// Here the threshold is exact rather than sampled. The indexer leaves, for
// each row, the counts of its scores over the top 12 bits of their
// order-preserving keys (hist[r][b] = #{s < L : order_key(score[s]) >> 20 ==
// b}). The bin where the count from the top first reaches k holds the k-th
// largest key: every key of a higher bin is selected and only that bin's
// keys need ranking, so no row can miss the threshold and nothing falls back
// to another method:
//   1. one block scan of the histogram row gives the threshold bin, the keys
//      above it and the keys in it (while the row's keys load); the
//      histogram row is cleared for the next step;
//   2. while the keys at or above the threshold prefix would not fit the
//      workgroup's LDS list, a radix pass over the row narrows the prefix by
//      12 more bits (re-reading rows longer than the registers hold);
//   3. one pass over the row compacts the keys at or above the prefix, with
//      their positions, into the LDS list in position order -- for a long
//      row the only read besides the narrowing passes;
//   4. radix passes over the list (a few keys per thread) finish the
//      threshold key and how many of the keys equal to it are needed;
//   5. an ordered compaction of the list writes the selection in ascending
//      position order, keys equal to the threshold taken in position order
//      ("ties to the lower position").
// If the bits run out, or the keys tied with the prefix are exactly those
// still needed, before the list is built, step 5 walks the row instead.
// Rows with L <= k take every position. Results are the same bits as
// dsa_topk's.

#include "radix_select.h"

namespace dsa {

template <int kThreads, int kVPT, int kCap>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ row_len,
                                                            uint32_t* __restrict__ hist, int width,
                                                            int k, int32_t* __restrict__ idx) {
  constexpr int kWaves = kThreads / 64;
  constexpr int kChunk = kThreads * kVPT;
  constexpr int kBPT = kHistBins / kThreads;  // histogram bins per thread
  constexpr int kEPT = kCap / kThreads;       // list entries per thread
  static_assert(kBPT % 4 == 0 && kEPT >= 1 && kEPT <= 32, "workgroup shape");
  typedef typename std::conditional<(kVPT <= 32), uint32_t, uint64_t>::type Mask;
  __shared__ uint32_t hbuf[2][kBins];           // radix-pass histograms, alternating
  __shared__ uint32_t scan_sh[3][kWaves];       // per-wave words: passes (2), histogram row (1)
  __shared__ uint32_t emit_sh[2][2 * kWaves];   // per-wave words of the compaction / emit scans
  __shared__ uint32_t pick[3];
  __shared__ uint32_t red[2 * kWaves];          // per-wave OR / AND of the list's candidates
  __shared__ uint32_t lkey[kCap];               // the list: keys at or above the prefix ...
  __shared__ int32_t lpos[kCap];                // ... and their positions, in position order

  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int L = row_len[r];
  int32_t* out = idx + (size_t)r * k;
  if (tid == 0) pick[0] = pick[1] = pick[2] = 0u;  // ordered before any reader by the scans below

  // 1a. The histogram row: thread t holds the bins of descending ranks
  // t*kBPT .. t*kBPT + kBPT - 1 (bin = kHistBins - 1 - rank); read, then
  // cleared.
  uint32_t hc[kBPT];
  {
    uint32_t* hrow = hist + (size_t)r * kHistBins + (kHistBins - (tid + 1) * kBPT);
#pragma unroll
    for (int i = 0; i < kBPT; i += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(hrow + i);
      hc[kBPT - 1 - i] = v.x;
      hc[kBPT - 2 - i] = v.y;
      hc[kBPT - 3 - i] = v.z;
      hc[kBPT - 4 - i] = v.w;
      *reinterpret_cast<uint4*>(hrow + i) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (L <= k) {
    for (int i = tid; i < k; i += kThreads) out[i] = i < L ? i : -1;
    return;
  }

  const float* row = scores + (size_t)r * width;
  const int nchunks = (L + kChunk - 1) / kChunk;
  const bool resident = (nchunks == 1);
  uint32_t key[kVPT];
  int nv = 0;
  auto load_chunk = [&](int c) {
    const int base = c * kChunk + tid * kVPT;
    nv = min(kVPT, max(0, L - base));
    if (nv == kVPT) {
#pragma unroll
      for (int j = 0; j < kVPT; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(row + base + j);
        key[j] = order_key(v.x);
        key[j + 1] = order_key(v.y);
        key[j + 2] = order_key(v.z);
        key[j + 3] = order_key(v.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kVPT; ++j) key[j] = (j < nv) ? order_key(row[base + j]) : 0u;
    }
  };
  if (resident) load_chunk(0);
  for (int i = tid; i < kBins; i += kThreads) hbuf[0][i] = 0u;  // while the keys arrive

  // 1b. The threshold bin: where the count from the top reaches k.
  uint32_t hsum = 0;
#pragma unroll
  for (int j = 0; j < kBPT; ++j) hsum += hc[j];
  uint32_t total;
  const uint32_t before = block_exclusive_scan<kWaves>(hsum, scan_sh[2], &total);
  if (before < (uint32_t)k && (uint32_t)k <= before + hsum) {
    uint32_t run = before;
    bool found = false;
#pragma unroll
    for (int j = 0; j < kBPT; ++j) {
      if (!found && run + hc[j] >= (uint32_t)k) {
        pick[0] = (uint32_t)(kHistBins - 1 - (tid * kBPT + j));
        pick[1] = run;
        pick[2] = hc[j];
        found = true;
      }
      run += hc[j];
    }
  }
  __syncthreads();
  int shift = kHistShift;
  uint32_t prefix = pick[0];
  uint32_t need = (uint32_t)k - pick[1];
  uint32_t cand = pick[2];
  if (total != (uint32_t)L) {
    // Not this row's histogram (a broken caller contract): rank from scratch,
    // which stays exact and in bounds.
    shift = 32;
    prefix = 0u;
    need = (uint32_t)k;
    cand = (uint32_t)L;
  }

  // One radix pass: the next <= 12 bits of the keys tied with the prefix.
  // `count` adds this thread's candidates to the histogram h.
  int hb = 0;
  int low = 0;  // the passes stop at this bit (see step 4)
  auto radix_pass = [&](auto&& count) {
    const int nb = min(kDigitBits, shift - low);
    const int ns = shift - nb;
    const int nbins = 1 << nb;
    uint32_t* h = hbuf[hb];
    count(h, ns, (uint32_t)nbins - 1u);
    for (int i = tid; i < kBins; i += kThreads) hbuf[hb ^ 1][i] = 0u;
    __syncthreads();
    constexpr int kMaxBpt = (kBins + kThreads - 1) / kThreads;
    const int bpt = (nbins + kThreads - 1) / kThreads;
    uint32_t cnt[kMaxBpt];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kMaxBpt; ++i) {
      const int rank = tid * bpt + i;
      cnt[i] = (i < bpt && rank < nbins) ? h[nbins - 1 - rank] : 0u;
      local += cnt[i];
    }
    uint32_t tot;
    const uint32_t bef = block_exclusive_scan<kWaves>(local, scan_sh[hb], &tot);
    if (bef < need && need <= bef + local) {
      uint32_t run = bef;
      bool found = false;
#pragma unroll
      for (int i = 0; i < kMaxBpt; ++i) {
        if (!found && run + cnt[i] >= need) {
          pick[0] = (uint32_t)(nbins - 1 - (tid * bpt + i));
          pick[1] = run;
          pick[2] = cnt[i];
          found = true;
        }
        run += cnt[i];
      }
    }
    __syncthreads();
    prefix = (prefix << nb) | pick[0];
    shift = ns;
    need -= pick[1];
    cand = pick[2];
    hb ^= 1;
  };

  // 2. Narrow while the keys at or above the prefix overflow the list.
  bool done = cand == need;
  while (!done && shift > 0 && (uint32_t)k - need + cand > (uint32_t)kCap) {
    // The chunks are re-read from cache even when one chunk holds the row:
    // keeping its keys live across this rarely taken loop would cost the
    // whole kernel registers.
    radix_pass([&](uint32_t* h, int ns, uint32_t dmask) {
      for (int c = 0; c < nchunks; ++c) {
        load_chunk(c);
#pragma unroll
        for (int j = 0; j < kVPT; ++j)
          if (j < nv && high_bits(key[j], shift) == prefix) atomicAdd(&h[(key[j] >> ns) & dmask], 1u);
      }
    });
    done = cand == need;
  }

  // An ordered compaction: each thread's items i < n in order, `gt` ones all
  // taken, `eq` ones taken while `need` lasts; one block scan of both counts
  // gives every thread its first output slots.
  auto emit = [&](uint32_t gt_run, uint32_t eq_run, auto gtm, auto eqm, auto&& pos_of,
                  uint32_t* words, uint32_t* gt_tot, uint32_t* eq_tot) {
    uint32_t xg, xe;
    block_exclusive_scan2<kWaves>((uint32_t)popcount(gtm), (uint32_t)popcount(eqm), words, &xg,
                                  &xe, gt_tot, eq_tot);
    uint32_t g = gt_run + xg, e = eq_run + xe;
    auto m = gtm | eqm;
    while (m) {
      const int j = lowest_bit(m);
      m &= m - 1;
      if ((gtm >> j) & 1) {
        const uint32_t slot = g + min(e, need);
        if (slot < (uint32_t)k) out[slot] = pos_of(j);
        ++g;
      } else {
        if (e < need && g + e < (uint32_t)k) out[g + e] = pos_of(j);
        ++e;
      }
    }
  };

  if (!done && shift > 0) {
    // 3. The keys at or above the prefix, in position order, into the list
    // (k - need + cand of them, at most kCap).
    uint32_t nlist = 0;
    for (int c = 0; c < nchunks; ++c) {
      if (!resident) load_chunk(c);
      const int base = c * kChunk + tid * kVPT;
      Mask m = 0;
#pragma unroll
      for (int j = 0; j < kVPT; ++j) m |= (Mask)(j < nv && high_bits(key[j], shift) >= prefix) << j;
      uint32_t tot;
      uint32_t o = nlist + block_exclusive_scan<kWaves>((uint32_t)popcount(m), emit_sh[c & 1], &tot);
      // A static walk over the thread's keys (indexing key[] by a bit found
      // at run time would move the array out of registers; re-reading the
      // score instead costs a dependent load per kept key).
#pragma unroll
      for (int j = 0; j < kVPT; ++j) {
        if ((m >> j) & 1) {
          if (o < (uint32_t)kCap) {
            lkey[o] = key[j];
            lpos[o] = base + j;
          }
          ++o;
        }
      }
      nlist += tot;
    }
    __syncthreads();
    // 4. Thread t holds list entries [t*kEPT, t*kEPT + kEPT).
    const int nl = (int)min(nlist, (uint32_t)kCap);
    const int e0 = tid * kEPT;
    const int ne = min(kEPT, max(0, nl - e0));
    uint32_t lk[kEPT];
#pragma unroll
    for (int j = 0; j < kEPT; ++j) lk[j] = j < ne ? lkey[e0 + j] : 0u;
    if (!done) {
      // Bits below the lowest one where two candidates differ are shared by
      // all of them (the trailing zeros of short dyadic significands, say):
      // the passes stop there, where equal prefixes mean equal keys.
      uint32_t oa = 0u, aa = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < kEPT; ++j)
        if (j < ne && high_bits(lk[j], shift) == prefix) {
          oa |= lk[j];
          aa &= lk[j];
        }
      wave_or_and(oa, aa);
      const int lane = tid & 63, wave = tid >> 6;
      if (lane == 0) {
        red[wave] = oa;
        red[kWaves + wave] = aa;
      }
      __syncthreads();
      oa = 0u;
      aa = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        oa |= red[i];
        aa &= red[kWaves + i];
      }
      // All candidates equal: no pass is left, the ties go by position.
      low = (oa ^ aa) ? min(shift, __ffs(oa ^ aa) - 1) : shift;
    }
    while (!done && shift > low) {
      radix_pass([&](uint32_t* h, int ns, uint32_t dmask) {
#pragma unroll
        for (int j = 0; j < kEPT; ++j)
          if (j < ne && high_bits(lk[j], shift) == prefix) atomicAdd(&h[(lk[j] >> ns) & dmask], 1u);
      });
      done = cand == need;
    }
    // 5. The selection from the list.
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
      const uint32_t hk = high_bits(lk[j], shift);
      gtm |= (uint32_t)(j < ne && hk > prefix) << j;
      eqm |= (uint32_t)(j < ne && hk == prefix) << j;
    }
    uint32_t tg, te;
    emit(0u, 0u, gtm, eqm, [&](int j) { return lpos[e0 + j]; }, emit_sh[0], &tg, &te);
    return;
  }

  // 5'. The selection from the row.
  uint32_t gt_run = 0, eq_run = 0;
  for (int c = 0; c < nchunks; ++c) {
    if (!resident) load_chunk(c);
    const int base = c * kChunk + tid * kVPT;
    Mask gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const uint32_t hk = high_bits(key[j], shift);
      gtm |= (Mask)(j < nv && hk > prefix) << j;
      eqm |= (Mask)(j < nv && hk == prefix) << j;
    }
    uint32_t tg, te;
    emit(gt_run, eq_run, gtm, eqm, [&](int j) { return base + j; }, emit_sh[c & 1], &tg, &te);
    gt_run += tg;
    eq_run += te;
  }
}

// Counts of each row's scores over the top 12 bits of their order keys,
// added to hist[r] (which the caller has cleared). Workgroup (r, g) of the G
// per row counts the row's chunks g, g + G, ... of kHistChunk positions; a
// thread loads its 32 consecutive scores of a chunk (eight 16-byte loads in
// flight) before counting them. A row's scores crowd into a few bins, and
// LDS atomics of one instruction to one address serialize, so lane l counts
// into copy l % kHistCopies of the histogram (16-bit counters, two bins a
// word); the copies are summed when the bins join the row's, one global
// atomic per non-empty bin. A copy takes 64 threads x 32 keys per chunk, so
// a workgroup counts at most kHistMaxIters chunks (the launch sets G).
constexpr int kHistThreads = 256;
constexpr int kHistVPT = 32;
constexpr int kHistChunk = kHistThreads * kHistVPT;  // 8192
constexpr int kHistCopies = 4;
constexpr int kHistMaxIters = 65535 / (kHistThreads / kHistCopies * kHistVPT);  // 31
constexpr int kHistWords = kHistBins / 2;  // per copy

__global__ __launch_bounds__(kHistThreads) void score_hist_kernel(const float* __restrict__ scores,
                                                                 const int32_t* __restrict__ row_len,
                                                                 int width, int groups,
                                                                 uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kHistCopies * kHistWords];
  const int r = blockIdx.x / groups;
  const int g = blockIdx.x - r * groups;
  const int L = row_len[r];
  if (g * kHistChunk >= L) return;  // uniform over the workgroup
  for (int i = threadIdx.x; i < kHistCopies * kHistWords; i += kHistThreads) h[i] = 0u;
  __syncthreads();
  const float* row = scores + (size_t)r * width;
  uint32_t* hc = h + (threadIdx.x % kHistCopies) * kHistWords;
  auto count = [&](float x) {
    const uint32_t bin = order_key(x) >> kHistShift;
    atomicAdd(&hc[bin >> 1], 1u << ((bin & 1u) << 4));
  };
  for (int c0 = g * kHistChunk; c0 < L; c0 += groups * kHistChunk) {
    const int p = c0 + (int)threadIdx.x * kHistVPT;
    if (p + kHistVPT <= L) {
      float4 v[kHistVPT / 4];
#pragma unroll
      for (int u = 0; u < kHistVPT / 4; ++u) v[u] = *reinterpret_cast<const float4*>(row + p + 4 * u);
#pragma unroll
      for (int u = 0; u < kHistVPT / 4; ++u) {
        count(v[u].x);
        count(v[u].y);
        count(v[u].z);
        count(v[u].w);
      }
    } else {
      for (int j = p; j < L; ++j) count(row[j]);
    }
  }
  __syncthreads();
  uint32_t* hr = hist + (size_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistWords; i += kHistThreads) {
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) {
      const uint32_t n = h[c * kHistWords + i];
      lo += n & 0xFFFFu;
      hi += n >> 16;
    }
    if (lo) atomicAdd(&hr[2 * i], lo);
    if (hi) atomicAdd(&hr[2 * i + 1], hi);
  }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_score_hist(const float* scores, const int32_t* row_len, int rows, int width,
                             uint32_t* hist, bool clear, hipStream_t stream) {
  if (clear) {
    const long long n = (long long)rows * kHistBins;
    const long long want = (n + 255) / 256;
    const int blocks = (int)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, stream, hist, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Workgroups per row: about four per compute unit over the batch, at most
  // one per chunk, and enough that none counts more than kHistMaxIters
  // chunks (its 16-bit counters).
  int cus = device_cus();
  if (cus <= 0) cus = 256;
  const int chunks = (width + kHistChunk - 1) / kHistChunk;
  const long long want = (4LL * cus + rows - 1) / rows;
  int groups = (int)(want < chunks ? want : chunks);
  const int least = (chunks + kHistMaxIters - 1) / kHistMaxIters;
  if (groups < least) groups = least;
  if (groups < 1) groups = 1;
  hipLaunchKernelGGL(score_hist_kernel, dim3((unsigned)((long long)rows * groups)),
                     dim3(kHistThreads), 0, stream, scores, row_len, width, groups, hist);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float* scores, const int32_t* row_len, uint32_t* hist, int rows,
                            int width, int k, int32_t* idx, hipStream_t stream,
                            long long total_keys) {
  // The workgroup shapes of launch_topk for narrow rows and batches of many
  // short rows (512 threads); everything wider runs 1024 threads x 32 keys:
  // a row longer than the registers hold is read once more for its list
  // rather than once per radix pass, so the 64-keys-per-thread shape (which
  // would spill here) is not needed. The list holds 8 keys per thread.
  int cus = device_cus();
  if (cus <= 0) cus = 256;
  const bool many_short = total_keys > 0 && rows >= 4 * cus && total_keys <= 16384LL * rows;
#define DSA_TOPK_HIST(T, V)                                                                    \
  hipLaunchKernelGGL((topk_hist_kernel<T, V, T * 8>), dim3(rows), dim3(T), 0, stream, scores, \
                     row_len, hist, width, k, idx)
  if (width <= 512 * 8) DSA_TOPK_HIST(512, 8);
  else if (width <= 512 * 16 || many_short) DSA_TOPK_HIST(512, 16);
  else if (width <= 512 * 32) DSA_TOPK_HIST(512, 32);
  else DSA_TOPK_HIST(1024, 32);
#undef DSA_TOPK_HIST
  return hipGetLastError();
}

}  // namespace dsa
