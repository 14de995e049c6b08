// Length-bounded exact top-k (Megatron-LM pull request 7211: commit "Replace
// the CuTe decode kernels with two Triton kernels" reads each row only up to
// its length; commit "When a step's context bound reaches 64K keys ..." keeps
// the result the exact top k; commit "Replace the Triton radix selector with
// torch.topk ..." ranks valid -inf scores ahead of padding).
//
// Row r with L = row_len[r] > k: select the k positions of [0, L) with the
// largest scores, ties to the lower position, and write them in ascending
// order. L <= k: every position, then -1.
//
// One workgroup per row: 512 threads for rows up to 16384 positions, else
// 1024; a thread owns up to 32 (or, for batches of few rows wider than 32768,
// 64) consecutive positions of each chunk, held in registers as
// order-preserving 32-bit keys (-0.0 canonicalized to +0.0).
// The threshold key is found by radix select on those keys:
//   * a min/max reduction skips the bits every key shares, so the first
//     12-bit digit falls where the row's values actually differ (scores of a
//     row usually share sign and leading exponent bits, which would otherwise
//     pile every key into one or two bins);
//   * each pass histograms the next <= 12 bits of the keys still tied with
//     the threshold prefix (LDS atomics; two buffers, so the next pass's is
//     cleared while this one is read) and a block scan over the bins, from
//     the top, picks the digit holding the k-th largest;
//   * it stops when the bits run out or every key still tied is needed.
// The emit pass is an ordered compaction: each thread counts its keys above
// the threshold prefix and equal to it, one block-wide exclusive scan of both
// counts (each a full 32-bit sum) gives every thread its output offsets, and keys equal to the prefix are taken in
// position order until the remaining need is met -- which is exactly
// "ties to the lower position". Rows longer than a chunk re-read their
// chunks from cache on every pass. Wave reductions and scans use DPP row
// operations and lane reads rather than LDS permutes, and every block scan
// has its own per-wave words, so a radix pass takes three barriers.

#include "radix_select.h"

namespace dsa {

// What one workgroup selects from.
enum TopkMode {
  kWholeRow = 0,  // row blockIdx.x, positions [0, row_len)
  kSegment = 1,   // segment c of row r (blockIdx.x = r * nseg + c): positions
                  // [c * seg, min(row_len, (c + 1) * seg)); winners' positions
                  // to idx + blockIdx.x * k, their keys to aux + blockIdx.x * k
  kGather = 2,    // row blockIdx.x over its segments' winners: positions at
                  // aux[row][nseg * k], their keys nseg * k * gridDim.x words
                  // further, the valid prefix of each; output the chosen
                  // positions
};

template <int kThreads, int kVPT, int kMode = kWholeRow>
// 512-thread workgroups keep two per compute unit: four waves per SIMD, so at
// most 128 registers (the second bound is waves per SIMD, not workgroups).
__global__ __launch_bounds__(kThreads, kThreads == 512 ? 4 : 1) void topk_kernel(const float* __restrict__ scores,
                                                       const int32_t* __restrict__ row_len,
                                                       int width, int k,
                                                       int32_t* __restrict__ idx, int seg,
                                                       int nseg, int32_t* __restrict__ aux) {
  constexpr int kTopkThreads = kThreads;
  constexpr int kTopkWaves = kThreads / 64;
  constexpr int kChunk = kThreads * kVPT;
  // One bit per position a thread owns in a chunk.
  typedef typename std::conditional<(kVPT <= 32), uint32_t, uint64_t>::type Mask;
  static_assert(kVPT <= 64, "a thread's positions must fit one 64-bit mask");
  __shared__ uint32_t hist[2][kBins];  // alternate passes: one fills while the other is cleared
  __shared__ uint32_t scan_sh[2][kTopkWaves];      // per-wave words of the radix passes' scans
  __shared__ uint32_t emit_sh[2][2 * kTopkWaves];  // ... and of the emit's, by chunk parity
  __shared__ uint32_t red[4 * kTopkWaves];
  __shared__ uint32_t pick[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // L: keys this workgroup selects from; pos0: position of its first key
  // (segment mode); gat: the candidate positions (gather mode).
  int r, L, pos0 = 0;
  const int32_t* gat = nullptr;     // gather mode: the candidates' positions
  const uint32_t* gkey = nullptr;   // ... and their keys
  uint32_t* outk = nullptr;         // segment mode: the winners' keys
  int32_t* out;
  if constexpr (kMode == kSegment) {
    r = (int)blockIdx.x / nseg;
    pos0 = ((int)blockIdx.x - r * nseg) * seg;
    L = min(seg, max(0, row_len[r] - pos0));
    out = idx + (size_t)blockIdx.x * k;
    outk = reinterpret_cast<uint32_t*>(aux) + (size_t)blockIdx.x * k;
  } else {
    r = blockIdx.x;
    L = row_len[r];
    out = idx + (size_t)r * k;
    if constexpr (kMode == kGather) {
      // Every segment but a row's last gave k winners (seg >= k), so the
      // valid candidates are a prefix, in ascending position order.
      const int n = (L + seg - 1) / seg;
      L = n == 0 ? 0 : k * (n - 1) + min(k, L - (n - 1) * seg);
      gat = aux + (size_t)r * nseg * k;
      gkey = reinterpret_cast<const uint32_t*>(aux) + (size_t)gridDim.x * nseg * k +
             (size_t)r * nseg * k;
    }
  }
  // Position of key i of this workgroup.
  auto pos_of = [&](int i) -> int32_t {
    if constexpr (kMode == kGather) return gat[i];
    else return pos0 + i;
  };
  if (L <= k) {
    if constexpr (kMode == kSegment) {
      // Every position is a winner; padding is never read (stage 2 takes the
      // valid prefix), so a short or empty segment writes only its own.
      for (int i = tid; i < L; i += kTopkThreads) {
        out[i] = pos0 + i;
        outk[i] = order_key(scores[(size_t)r * width + pos0 + i]);
      }
    } else {
      for (int i = tid; i < k; i += kTopkThreads) out[i] = i < L ? pos_of(i) : -1;
    }
    return;
  }
  const float* row = scores + (size_t)r * width + pos0;
  const int nchunks = (L + kChunk - 1) / kChunk;
  uint32_t key[kVPT];
  int nv = 0;  // valid positions among this thread's kVPT in the current chunk

  // Keys of chunk c: positions c*kChunk + tid*kVPT + j; invalid ones read as 0
  // and are excluded by nv.
  auto load_chunk = [&](int c) {
    const int base = c * kChunk + tid * kVPT;
    nv = min(kVPT, max(0, L - base));
    if constexpr (kMode == kGather) {
      // The candidates' keys, written by stage 1 next to their positions.
#pragma unroll
      for (int j = 0; j < kVPT; ++j) key[j] = j < nv ? gkey[base + j] : 0u;
    } else if (nv == kVPT) {
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
  const bool resident = (nchunks == 1);
  if (resident) load_chunk(0);
  for (int i = tid; i < kBins; i += kTopkThreads) hist[0][i] = 0u;  // while the keys arrive

  // ---- min / max over the row, and the bits every key shares ----------------
  uint32_t mx = 0u, mn = 0xFFFFFFFFu, oa = 0u, aa = 0xFFFFFFFFu;
  for (int c = 0; c < nchunks; ++c) {
    if (!resident) load_chunk(c);
    if (nv == kVPT) {
#pragma unroll
      for (int j = 0; j < kVPT; ++j) {
        mx = max(mx, key[j]);
        mn = min(mn, key[j]);
        oa |= key[j];
        aa &= key[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kVPT; ++j)
        if (j < nv) {
          mx = max(mx, key[j]);
          mn = min(mn, key[j]);
          oa |= key[j];
          aa &= key[j];
        }
    }
  }
  wave_max_min(mx, mn);
  wave_or_and(oa, aa);
  if (lane == 0) {
    red[wave] = mx;
    red[kTopkWaves + wave] = mn;
    red[2 * kTopkWaves + wave] = oa;
    red[3 * kTopkWaves + wave] = aa;
  }
  __syncthreads();
  mx = 0u;
  mn = 0xFFFFFFFFu;
  oa = 0u;
  aa = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    mx = max(mx, red[i]);
    mn = min(mn, red[kTopkWaves + i]);
    oa |= red[2 * kTopkWaves + i];
    aa &= red[3 * kTopkWaves + i];
  }

  // ---- radix select of the threshold prefix --------------------------------
  // Candidates are the keys whose bits at and above `shift` equal `prefix`;
  // `need` of them are still to be taken, and every key above the prefix is
  // taken. Every key shares the bits above the highest bit where the row's
  // min and max differ, so the first digit starts there and needs no prefix
  // test.
  // Bits below the lowest one where any two keys differ are the same in every
  // key (the trailing zeros of short dyadic significands, say), so the
  // passes stop there: comparing the bits above it compares whole keys.
  int shift, low = 0;
  uint32_t prefix;
  uint32_t need = (uint32_t)k;
  if (mx == mn) {
    shift = 0;
    prefix = mx;
  } else {
    shift = 32 - __clz(mx ^ mn);
    prefix = high_bits(mx, shift);
    low = __ffs(oa ^ aa) - 1;
  }
  // Three barriers per pass: after the histogram, inside the bin scan, and
  // after the pick. The next pass's histogram buffer is cleared while this
  // one is read, and every scan has its own per-wave words.
  bool first = true;
  int hb = 0;
  while (shift > low) {
    const int nb = min(kDigitBits, shift - low);
    const int ns = shift - nb;
    const int nbins = 1 << nb;
    const uint32_t dmask = (uint32_t)nbins - 1u;
    uint32_t* h = hist[hb];
    for (int c = 0; c < nchunks; ++c) {
      if (!resident) load_chunk(c);
      if (first && nv == kVPT) {
#pragma unroll
        for (int j = 0; j < kVPT; ++j) atomicAdd(&h[(key[j] >> ns) & dmask], 1u);
      } else if (first) {
#pragma unroll
        for (int j = 0; j < kVPT; ++j)
          if (j < nv) atomicAdd(&h[(key[j] >> ns) & dmask], 1u);
      } else if (nv == kVPT) {
#pragma unroll
        for (int j = 0; j < kVPT; ++j)
          if ((key[j] >> shift) == prefix) atomicAdd(&h[(key[j] >> ns) & dmask], 1u);
      } else {
#pragma unroll
        for (int j = 0; j < kVPT; ++j)
          if (j < nv && (key[j] >> shift) == prefix) atomicAdd(&h[(key[j] >> ns) & dmask], 1u);
      }
    }
    // The other buffer was last read before the previous pass's final barrier.
    for (int i = tid; i < kBins; i += kTopkThreads) hist[hb ^ 1][i] = 0u;
    __syncthreads();
    // Bins in descending digit order; thread t owns ranks [t*bpt, t*bpt+bpt).
    constexpr int kMaxBpt = (kBins + kTopkThreads - 1) / kTopkThreads;
    const int bpt = (nbins + kTopkThreads - 1) / kTopkThreads;
    uint32_t cnt[kMaxBpt];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kMaxBpt; ++i) {
      const int rank = tid * bpt + i;
      cnt[i] = (i < bpt && rank < nbins) ? h[nbins - 1 - rank] : 0u;
      local += cnt[i];
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<kTopkWaves>(local, scan_sh[hb], &total);
    if (before < need && need <= before + local) {
      uint32_t run = before;
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
    // The next write of `pick` comes after two barriers of the next pass.
    __syncthreads();
    const uint32_t digit = pick[0], above = pick[1], cand = pick[2];
    prefix = (prefix << nb) | digit;
    shift = ns;
    need -= above;
    first = false;
    hb ^= 1;
    if (cand == need) break;
  }

  // ---- ordered emit ---------------------------------------------------------
  // Each thread marks its keys above the prefix (taken) and equal to it
  // (taken in position order while `need` lasts), one block scan of the two
  // counts gives its output offsets, and it walks only its marked keys.
  uint32_t gt_run = 0, eq_run = 0;
  for (int c = 0; c < nchunks; ++c) {
    if (!resident) load_chunk(c);
    const int base = c * kChunk + tid * kVPT;
    Mask gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const uint32_t hb = key[j] >> shift;
      gtm |= (Mask)(hb > prefix) << j;
      eqm |= (Mask)(hb == prefix) << j;
    }
    const Mask vmask = nv == kVPT ? ~(Mask)0 : (((Mask)1 << nv) - 1);
    gtm &= vmask;
    eqm &= vmask;
    uint32_t excl_gt, excl_eq, tot_gt, tot_eq;
    // Scans of consecutive chunks use different words; each scan's barrier
    // orders the reads of the one before.
    if constexpr (kChunk < 65536) {
      // Both counts of a chunk and their prefix sums stay below 65536, so
      // they share one word (one scan, fewer registers).
      uint32_t tot;
      const uint32_t ex = block_exclusive_scan<kTopkWaves>(
          ((uint32_t)popcount(gtm) << 16) | (uint32_t)popcount(eqm), emit_sh[c & 1], &tot);
      excl_gt = ex >> 16;
      excl_eq = ex & 0xffffu;
      tot_gt = tot >> 16;
      tot_eq = tot & 0xffffu;
    } else {
      block_exclusive_scan2<kTopkWaves>((uint32_t)popcount(gtm), (uint32_t)popcount(eqm),
                                        emit_sh[c & 1], &excl_gt, &excl_eq, &tot_gt, &tot_eq);
    }
    uint32_t g = gt_run + excl_gt;
    uint32_t e = eq_run + excl_eq;
    // The winners' keys (segment mode) are re-read from the row, a cache
    // hit: indexing key[] by the bit found at run time would move the whole
    // array out of registers.
    Mask m = gtm | eqm;
    while (m) {
      const int j = lowest_bit(m);
      m &= m - 1;
      // Every slot written is < k by construction; the bound keeps a broken
      // invariant from ever turning into an out-of-row store.
      if ((gtm >> j) & 1) {
        const uint32_t slot = g + min(e, need);
        if (slot < (uint32_t)k) {
          out[slot] = pos_of(base + j);
          if constexpr (kMode == kSegment) outk[slot] = order_key(row[base + j]);
        }
        ++g;
      } else {
        if (e < need && g + e < (uint32_t)k) {
          out[g + e] = pos_of(base + j);
          if constexpr (kMode == kSegment) outk[g + e] = order_key(row[base + j]);
        }
        ++e;
      }
    }
    gt_run += tot_gt;
    eq_run += tot_eq;
  }
}

hipError_t launch_topk(const float* scores, const int32_t* row_len, int rows, int width, int k,
                       int32_t* idx, hipStream_t stream, long long total_keys) {
  // 32 keys per thread cover rows up to 32768 positions in registers. Wider
  // batches of few rows (the long rows set the kernel's time) hold 64 keys per
  // thread, which halves the chunk re-reads of rows past 32768; batches of
  // many rows fill the device either way and keep 32 (shorter rows then use
  // more of the workgroup's threads).
  int cus = device_cus();
  if (cus <= 0) cus = 256;
  // Narrow rows: 512 threads holding up to 32 keys each. A radix pass costs
  // about the same in barriers and bin scans whatever the row length, and
  // with half the waves those fixed costs halve (batch 8, width 4096:
  // 15.0 -> 7.7 us); from 32768 positions the 1024-thread kernel is faster.
  // Batches of at least 4 rows per CU whose rows are short on average (the
  // host's total_keys hint) take 512 x 16 whatever the width: the rows fill
  // the device several times over, so small workgroups that many CUs hold at
  // once beat wide ones, and the few long rows re-read their chunks (mixed
  // prefill + decode step, 2108 rows, width 131072, mean length ~10K:
  // 219 -> 140 us; batch 64 ragged keeps the wide kernel, 32 vs 43 us).
  const bool many_short = total_keys > 0 && rows >= 4 * cus && total_keys <= 16384LL * rows;
  if (width <= 512 * 8) {
    hipLaunchKernelGGL((topk_kernel<512, 8>), dim3(rows), dim3(512), 0, stream, scores, row_len,
                       width, k, idx, 0, 1, nullptr);
    return hipGetLastError();
  }
  if (width <= 512 * 16 || many_short) {
    hipLaunchKernelGGL((topk_kernel<512, 16>), dim3(rows), dim3(512), 0, stream, scores, row_len,
                       width, k, idx, 0, 1, nullptr);
    return hipGetLastError();
  }
  if (width <= 512 * 32) {
    hipLaunchKernelGGL((topk_kernel<512, 32>), dim3(rows), dim3(512), 0, stream, scores, row_len,
                       width, k, idx, 0, 1, nullptr);
    return hipGetLastError();
  }
  if (width > kTopkThreads * 32 && rows <= cus)
    hipLaunchKernelGGL((topk_kernel<kTopkThreads, 64>), dim3(rows), dim3(kTopkThreads), 0, stream,
                       scores, row_len, width, k, idx, 0, 1, nullptr);
  else
    hipLaunchKernelGGL((topk_kernel<kTopkThreads, 32>), dim3(rows), dim3(kTopkThreads), 0, stream,
                       scores, row_len, width, k, idx, 0, 1, nullptr);
  return hipGetLastError();
}

int topk_segments(int width, int seg) { return (width + seg - 1) / seg; }

int topk_suggest_chunk(int rows, int width, int k, bool full) {
  // One workgroup holds up to 64K keys of a row in registers; longer rows
  // re-read their chunks on every radix pass, so from there the two-stage
  // selection over 32768-position segments is faster -- for rows that fill
  // the width (`full`) at any batch size, otherwise (a few long rows among
  // short ones) as long as its first stage stays within a few workgroups per
  // compute unit.
  constexpr int kSeg = kTopkThreads * 32;
  int cus = device_cus();
  if (cus <= 0) cus = 256;
  if (width <= kTopkThreads * 64 || k > kSeg) return 0;
  if (full) return kSeg;
  const long long wgs = (long long)rows * topk_segments(width, kSeg);
  return wgs <= 4LL * cus ? kSeg : 0;
}

hipError_t launch_topk_chunked(const float* scores, const int32_t* row_len, int rows, int width,
                               int k, int seg, int32_t* cand, int32_t* idx, hipStream_t stream) {
  // Stage 1: the exact top-k of every segment of every row (a segment's
  // winners include every global winner that lies in it): positions into
  // the first half of cand, their keys into the second.
  const int nseg = topk_segments(width, seg);
  const long long wgs = (long long)rows * nseg;
  int32_t* keys = cand + (size_t)wgs * k;
  // Segments of up to 32768 positions run in 512-thread workgroups: the
  // stage has many of them, and smaller workgroups pay less in barriers per
  // radix pass (512 x 1M positions in 32768-position segments: 1490 ->
  // 1200 us against 1024 threads x 32 keys).
  if (seg <= 512 * 32)
    hipLaunchKernelGGL((topk_kernel<512, 32, kSegment>), dim3((unsigned)wgs), dim3(512), 0,
                       stream, scores, row_len, width, k, cand, seg, nseg, keys);
  else if (seg <= 512 * 64)
    hipLaunchKernelGGL((topk_kernel<512, 64, kSegment>), dim3((unsigned)wgs), dim3(512), 0,
                       stream, scores, row_len, width, k, cand, seg, nseg, keys);
  else
    hipLaunchKernelGGL((topk_kernel<kTopkThreads, 64, kSegment>), dim3((unsigned)wgs),
                       dim3(kTopkThreads), 0, stream, scores, row_len, width, k, cand, seg, nseg,
                       keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Stage 2: the exact top-k of each row over its segments' winners.
  if ((long long)nseg * k <= kTopkThreads * 32)
    hipLaunchKernelGGL((topk_kernel<kTopkThreads, 32, kGather>), dim3(rows), dim3(kTopkThreads), 0,
                       stream, scores, row_len, width, k, idx, seg, nseg, cand);
  else
    hipLaunchKernelGGL((topk_kernel<kTopkThreads, 64, kGather>), dim3(rows), dim3(kTopkThreads), 0,
                       stream, scores, row_len, width, k, idx, seg, nseg, cand);
  return hipGetLastError();
}

}  // namespace dsa
