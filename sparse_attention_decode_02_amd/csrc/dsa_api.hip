// C ABI of libdsa.so: host-side argument checks, row planning, and dispatch
// to the HIP kernels. Every check runs before any launch, so a negative
// status means nothing was enqueued and no output was touched. No entry
// point allocates, frees, synchronizes, or reads device memory.

#include <math.h>

#include <algorithm>
#include <atomic>

#include "../../include/dsa.h"
#include "dsa_kernels.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// log2 of a power of two in [1, 65536], else -1.
int pow2_shift(int v) {
  if (v < 1 || v > 65536 || (v & (v - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) != v) ++s;
  return s;
}

int launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

}  // namespace


namespace {

// Argument checks of dsa_indexer_scores; *page_shift gets log2(page_size).
int indexer_check(const void* q_idx, const float* w, const void* k_idx_cache,
                  const int32_t* block_table, const int32_t* row_req, const int32_t* row_len,
                  const int32_t* blocks, int num_blocks, const float* scores, int rows, int width,
                  int num_heads, int head_dim, int page_size, int max_pages, dsa_dtype dtype,
                  bool full, int* page_shift) {
  if (!q_idx || !w || !k_idx_cache || !block_table || !row_req || !row_len || !scores)
    return DSA_ERR_NULL;
  if (rows < 0 || width < 1 || (width & 3) != 0 || max_pages < 1) return DSA_ERR_SHAPE;
  const int ps = pow2_shift(page_size);
  if (ps < 0) return DSA_ERR_SHAPE;
  if (blocks && (num_blocks < 1 || num_blocks > rows)) return DSA_ERR_SHAPE;
  if (dtype == DSA_BF16) {
    if (!((head_dim == 128 || head_dim == 64) && (num_heads == 32 || num_heads == 64)) ||
        page_size < 16)
      return DSA_ERR_UNSUPPORTED;
  } else if (dtype == DSA_F32) {
    if (!((head_dim == 32 || head_dim == 64 || head_dim == 128) && num_heads >= 1 &&
          num_heads <= 64))
      return DSA_ERR_UNSUPPORTED;
  } else {
    return DSA_ERR_UNSUPPORTED;
  }
  if (!aligned(q_idx, 16) || !aligned(k_idx_cache, 16) || !aligned(scores, 16) || !aligned(w, 4) ||
      !aligned(block_table, 4) || !aligned(row_req, 4) || !aligned(row_len, 4) ||
      (blocks && !aligned(blocks, 4)))
    return DSA_ERR_ALIGN;
  const int nb = blocks ? num_blocks : rows;
  if (rows > 0 && dtype == DSA_BF16) {
    int chunk = dsa::indexer_chunk_keys(nb, width, num_heads, head_dim, full);
    if (blocks && dsa::indexer_uses_blocks(rows, nb))
      chunk = std::min(chunk, dsa::indexer_block_chunk_keys(nb, width, num_heads, head_dim, full));
    if ((long long)nb * ((width + chunk - 1) / chunk) > INT32_MAX - 64) return DSA_ERR_SHAPE;
  } else if (rows > 0 && (long long)nb * ((width + 255) / 256) > INT32_MAX) {
    return DSA_ERR_SHAPE;
  }
  *page_shift = ps;
  return DSA_OK;
}

hipError_t indexer_launch(const void* q_idx, const float* w, const void* k_idx_cache,
                          const int32_t* block_table, const int32_t* row_req,
                          const int32_t* row_len, const int32_t* blocks, int num_blocks,
                          float* scores, int rows, int width, int num_heads, int head_dim,
                          int page_shift, int max_pages, dsa_dtype dtype, bool full,
                          hipStream_t st, int score_row0 = 0, uint32_t* hist = nullptr,
                          long long total_keys = 0) {
  const int nb = blocks ? num_blocks : rows;
  if (dtype == DSA_BF16)
    return dsa::launch_indexer_bf16(q_idx, w, k_idx_cache, block_table, row_req, row_len, blocks,
                                    nb, rows, scores, width, num_heads, head_dim, page_shift,
                                    max_pages, full, score_row0, st, hist, total_keys);
  hipError_t e = dsa::launch_indexer_f32(static_cast<const float*>(q_idx), w,
                                         static_cast<const float*>(k_idx_cache), block_table,
                                         row_req, row_len, blocks, nb, scores, width, num_heads,
                                         head_dim, page_shift, max_pages, score_row0, st);
  if (e == hipSuccess && hist)
    e = dsa::launch_score_hist(scores, row_len, rows, width, hist, false, st);
  return e;
}

int topk_check(const float* scores, const int32_t* row_len, int rows, int width, int k,
               const int32_t* idx) {
  if (!scores || !row_len || !idx) return DSA_ERR_NULL;
  if (rows < 0 || width < 1 || (width & 3) != 0 || k < 1 || k > width) return DSA_ERR_SHAPE;
  if (!aligned(scores, 16) || !aligned(row_len, 4) || !aligned(idx, 4)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

// Chunked top-k: chunk >= k, a multiple of 4 (segments start on 16-byte
// boundaries of the score row); *slots gets the int32 workspace slots
// needed (each segment winner's position and key).
int topk_chunked_check(int rows, int width, int k, int chunk, long long* slots) {
  if (rows < 0 || width < 1 || k < 1 || k > width) return DSA_ERR_SHAPE;
  if (chunk < k || (chunk & 3) != 0 || chunk > (1 << 20)) return DSA_ERR_SHAPE;
  const long long nseg = dsa::topk_segments(width, chunk);
  const long long s = 2LL * rows * nseg * k;  // positions, then their keys
  if ((long long)rows * nseg > INT32_MAX || s > (1LL << 40)) return DSA_ERR_SHAPE;
  *slots = s;
  return DSA_OK;
}

}  // namespace

// ---- The allocation-free two-stage top-k's workspace -----------------------
// dsa_topk_chunked_noalloc keeps the segment winners (positions, then keys)
// in this array instead of a caller-given buffer. Each device that loads the
// library holds its own copy until the process ends. In host code the name
// `scratch` stands for a host-side shadow, not device memory: only the device
// address looked up below (scratch_on_device) is ever passed to a kernel.
static __device__ __align__(256) int32_t scratch[DSA_TOPK_NOALLOC_MAX_SLOTS];

namespace {

constexpr int kMaxScratchDevices = 1024;
std::atomic<int32_t*> g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on device `dev` (the current device), looked up
// with hipGetSymbolAddress on the first call there and kept; NULL on failure.
int32_t* scratch_on_device(int dev) {
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
    return nullptr;
  p = static_cast<int32_t*>(addr);
  g_scratch_ptr[dev].store(p, std::memory_order_release);  // the same address if two threads race
  return p;
}

}  // namespace

extern "C" {

int dsa_topk_chunked_noalloc(const float* scores, const int32_t* row_len, int rows, int width,
                             int k, int chunk, int32_t* idx, void* stream) {
  int st = topk_check(scores, row_len, rows, width, k, idx);
  if (st != DSA_OK) return st;
  long long need = 0;
  st = topk_chunked_check(rows, width, k, chunk, &need);
  if (st != DSA_OK) return st;
  if (need > DSA_TOPK_NOALLOC_MAX_SLOTS) return DSA_ERR_WORKSPACE;
  if (rows == 0) return DSA_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return DSA_ERR_LAUNCH;
  int32_t* cand = scratch_on_device(dev);
  if (!cand) return DSA_ERR_LAUNCH;
  // Stage 1 writes every candidate stage 2 reads, so nothing is cleared.
  return launch_status(dsa::launch_topk_chunked(scores, row_len, rows, width, k, chunk, cand, idx,
                                                static_cast<hipStream_t>(stream)));
}

int dsa_indexer_scores_total(const void* q_idx, const float* w, const void* k_idx_cache,
                             const int32_t* block_table, const int32_t* row_req,
                             const int32_t* row_len, const int32_t* blocks, int num_blocks,
                             float* scores, int rows, int width, int num_heads, int head_dim,
                             int page_size, int max_pages, dsa_dtype dtype, long long total_keys,
                             void* stream) {
  if (total_keys < 0 || total_keys > (long long)rows * width) return DSA_ERR_SHAPE;
  // Rows that fill at least 90% of the score width have no ragged tail.
  const bool full = rows > 0 && total_keys * 10 >= (long long)rows * width * 9;
  int ps = 0;
  const int st = indexer_check(q_idx, w, k_idx_cache, block_table, row_req, row_len, blocks,
                               num_blocks, scores, rows, width, num_heads, head_dim, page_size,
                               max_pages, dtype, full, &ps);
  if (st != DSA_OK) return st;
  if (rows == 0) return DSA_OK;
  return launch_status(indexer_launch(q_idx, w, k_idx_cache, block_table, row_req, row_len,
                                      blocks, num_blocks, scores, rows, width, num_heads,
                                      head_dim, ps, max_pages, dtype, full,
                                      static_cast<hipStream_t>(stream), 0, nullptr, total_keys));
}

int dsa_indexer_scores_hist(const void* q_idx, const float* w, const void* k_idx_cache,
                            const int32_t* block_table, const int32_t* row_req,
                            const int32_t* row_len, const int32_t* blocks, int num_blocks,
                            float* scores, uint32_t* hist, int rows, int width, int num_heads,
                            int head_dim, int page_size, int max_pages, dsa_dtype dtype,
                            long long total_keys, void* stream) {
  if (!hist) return DSA_ERR_NULL;
  if (!aligned(hist, 16)) return DSA_ERR_ALIGN;
  if (total_keys < 0 || total_keys > (long long)rows * width) return DSA_ERR_SHAPE;
  const bool full = rows > 0 && total_keys * 10 >= (long long)rows * width * 9;
  int ps = 0;
  const int st = indexer_check(q_idx, w, k_idx_cache, block_table, row_req, row_len, blocks,
                               num_blocks, scores, rows, width, num_heads, head_dim, page_size,
                               max_pages, dtype, full, &ps);
  if (st != DSA_OK) return st;
  if (rows == 0) return DSA_OK;
  return launch_status(indexer_launch(q_idx, w, k_idx_cache, block_table, row_req, row_len,
                                      blocks, num_blocks, scores, rows, width, num_heads,
                                      head_dim, ps, max_pages, dtype, full,
                                      static_cast<hipStream_t>(stream), 0, hist, total_keys));
}

int dsa_indexer_scores(const void* q_idx, const float* w, const void* k_idx_cache,
                       const int32_t* block_table, const int32_t* row_req, const int32_t* row_len,
                       const int32_t* blocks, int num_blocks, float* scores, int rows, int width,
                       int num_heads, int head_dim, int page_size, int max_pages, dsa_dtype dtype,
                       void* stream) {
  return dsa_indexer_scores_total(q_idx, w, k_idx_cache, block_table, row_req, row_len, blocks,
                                  num_blocks, scores, rows, width, num_heads, head_dim, page_size,
                                  max_pages, dtype, 0, stream);
}

int dsa_topk(const float* scores, const int32_t* row_len, int rows, int width, int k,
             int32_t* idx, void* stream) {
  const int st = topk_check(scores, row_len, rows, width, k, idx);
  if (st != DSA_OK) return st;
  if (rows == 0) return DSA_OK;
  return launch_status(
      dsa::launch_topk(scores, row_len, rows, width, k, idx, static_cast<hipStream_t>(stream)));
}

int dsa_topk_total(const float* scores, const int32_t* row_len, int rows, int width, int k,
                   long long total_keys, int32_t* idx, void* stream) {
  if (total_keys < 0 || total_keys > (long long)rows * width) return DSA_ERR_SHAPE;
  const int st = topk_check(scores, row_len, rows, width, k, idx);
  if (st != DSA_OK) return st;
  if (rows == 0) return DSA_OK;
  return launch_status(dsa::launch_topk(scores, row_len, rows, width, k, idx,
                                        static_cast<hipStream_t>(stream), total_keys));
}

int dsa_topk_hist(const float* scores, const int32_t* row_len, uint32_t* hist, int rows,
                  int width, int k, long long total_keys, int32_t* idx, void* stream) {
  if (total_keys < 0 || total_keys > (long long)rows * width) return DSA_ERR_SHAPE;
  const int st = topk_check(scores, row_len, rows, width, k, idx);
  if (st != DSA_OK) return st;
  if (!hist) return DSA_ERR_NULL;
  if (!aligned(hist, 16)) return DSA_ERR_ALIGN;
  if (rows == 0) return DSA_OK;
  return launch_status(dsa::launch_topk_hist(scores, row_len, hist, rows, width, k, idx,
                                             static_cast<hipStream_t>(stream), total_keys));
}

int dsa_score_hist(const float* scores, const int32_t* row_len, int rows, int width,
                   uint32_t* hist, void* stream) {
  if (!scores || !row_len || !hist) return DSA_ERR_NULL;
  if (rows < 0 || width < 1) return DSA_ERR_SHAPE;
  if ((long long)rows * ((width + 8191) / 8192) > INT32_MAX) return DSA_ERR_SHAPE;
  if (!aligned(scores, 4) || !aligned(row_len, 4) || !aligned(hist, 16)) return DSA_ERR_ALIGN;
  if (rows == 0) return DSA_OK;
  return launch_status(dsa::launch_score_hist(scores, row_len, rows, width, hist, true,
                                              static_cast<hipStream_t>(stream)));
}

int dsa_topk_chunked_slots(int rows, int width, int k, int chunk, long long* slots) {
  if (!slots) return DSA_ERR_NULL;
  return topk_chunked_check(rows, width, k, chunk, slots);
}

int dsa_topk_chunked(const float* scores, const int32_t* row_len, int rows, int width, int k,
                     int chunk, int32_t* cand, long long cand_slots, int32_t* idx, void* stream) {
  int st = topk_check(scores, row_len, rows, width, k, idx);
  if (st != DSA_OK) return st;
  if (!cand) return DSA_ERR_NULL;
  long long need = 0;
  st = topk_chunked_check(rows, width, k, chunk, &need);
  if (st != DSA_OK) return st;
  if (cand_slots < need) return DSA_ERR_WORKSPACE;
  if (!aligned(cand, 4)) return DSA_ERR_ALIGN;
  if (rows == 0) return DSA_OK;
  return launch_status(dsa::launch_topk_chunked(scores, row_len, rows, width, k, chunk, cand, idx,
                                                static_cast<hipStream_t>(stream)));
}

int dsa_topk_chunk_suggest(int rows, int width, int k, long long total_keys, int* chunk) {
  if (!chunk) return DSA_ERR_NULL;
  if (rows < 0 || width < 1 || k < 1 || k > width) return DSA_ERR_SHAPE;
  if (total_keys < 0 || total_keys > (long long)rows * width) return DSA_ERR_SHAPE;
  const bool full = rows > 0 && total_keys * 10 >= (long long)rows * width * 9;
  *chunk = dsa::topk_suggest_chunk(rows, width, k, full);
  return DSA_OK;
}


// Windows over a score-block plan: each window is a run of whole blocks
// holding at most `window` rows. blocks_host must cover rows 0..rows-1 in
// order; a block longer than a window cannot be placed.
static int plan_block_windows(const int32_t* blocks, int num_blocks, int rows, int window) {
  int next = 0;
  for (int b = 0; b < num_blocks; ++b) {
    const int first = blocks[2 * b], n = blocks[2 * b + 1];
    if (first != next || n < 1 || n > rows - next) return DSA_ERR_SHAPE;
    if (n > window) return DSA_ERR_WORKSPACE;
    next += n;
  }
  return next == rows ? DSA_OK : DSA_ERR_SHAPE;
}

int dsa_indexer_topk_windowed(const void* q_idx, const float* w, const void* k_idx_cache,
                              const int32_t* block_table, const int32_t* row_req,
                              const int32_t* row_len, const int32_t* blocks_host,
                              const int32_t* blocks_dev, int num_blocks, int rows, int width,
                              int num_heads, int head_dim, int page_size, int max_pages,
                              dsa_dtype dtype, int k, float* score_buffer,
                              long long score_buffer_bytes, int topk_chunk, int32_t* cand,
                              long long cand_slots, int32_t* idx, void* stream) {
  int window = 0;
  int st = dsa_select_window_rows(width, score_buffer_bytes, &window);
  if (st != DSA_OK) return st;
  if (rows < 0) return DSA_ERR_SHAPE;
  if (window > rows) window = rows;
  const bool with_blocks = num_blocks > 0;
  if (with_blocks) {
    if (!blocks_host || !blocks_dev) return DSA_ERR_NULL;
    if (num_blocks > rows) return DSA_ERR_SHAPE;
    st = plan_block_windows(blocks_host, num_blocks, rows, window);
    if (st != DSA_OK) return st;
  } else if (num_blocks < 0) {
    return DSA_ERR_SHAPE;
  }
  // Every window passes the checks of the whole call: row offsets keep the
  // alignments (a query row is a multiple of 16 bytes).
  int ps = 0;
  st = indexer_check(q_idx, w, k_idx_cache, block_table, row_req, row_len,
                     with_blocks ? blocks_dev : nullptr, num_blocks, score_buffer,
                     with_blocks ? rows : window, width, num_heads, head_dim, page_size,
                     max_pages, dtype, false, &ps);
  if (st != DSA_OK) return st;
  st = topk_check(score_buffer, row_len, window, width, k, idx);
  if (st != DSA_OK) return st;
  if (topk_chunk > 0) {
    if (!cand) return DSA_ERR_NULL;
    long long need = 0;
    st = topk_chunked_check(window, width, k, topk_chunk, &need);
    if (st != DSA_OK) return st;
    if (cand_slots < need) return DSA_ERR_WORKSPACE;
    if (!aligned(cand, 4)) return DSA_ERR_ALIGN;
  } else if (topk_chunk < 0) {
    return DSA_ERR_SHAPE;
  }
  if (rows == 0) return DSA_OK;
  const size_t qrow = (size_t)num_heads * head_dim * (dtype == DSA_BF16 ? 2 : 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Both launches of a window go to one stream, so the next window's scores
  // overwrite the buffer only after this window's selection has read it.
  auto select = [&](int r0, int n) {
    return topk_chunk > 0 ? dsa::launch_topk_chunked(score_buffer, row_len + r0, n, width, k,
                                                      topk_chunk, cand, idx + (size_t)r0 * k, s)
                          : dsa::launch_topk(score_buffer, row_len + r0, n, width, k,
                                             idx + (size_t)r0 * k, s);
  };
  if (with_blocks) {
    // Whole blocks per window; the kernel reads rows at their own index and
    // writes scores from the window's first row.
    for (int b0 = 0; b0 < num_blocks;) {
      const int r0 = blocks_host[2 * b0];
      int b1 = b0, n = 0;
      while (b1 < num_blocks && n + blocks_host[2 * b1 + 1] <= window) n += blocks_host[2 * b1++ + 1];
      hipError_t e = indexer_launch(q_idx, w, k_idx_cache, block_table, row_req, row_len,
                                    blocks_dev + 2 * (size_t)b0, b1 - b0, score_buffer, n, width,
                                    num_heads, head_dim, ps, max_pages, dtype, false, s, r0);
      if (e != hipSuccess) return DSA_ERR_LAUNCH;
      if (select(r0, n) != hipSuccess) return DSA_ERR_LAUNCH;
      b0 = b1;
    }
    return DSA_OK;
  }
  for (int r0 = 0; r0 < rows; r0 += window) {
    const int n = rows - r0 < window ? rows - r0 : window;
    hipError_t e = indexer_launch(static_cast<const char*>(q_idx) + (size_t)r0 * qrow,
                                  w + (size_t)r0 * num_heads, k_idx_cache, block_table,
                                  row_req + r0, row_len + r0, nullptr, 0, score_buffer, n, width,
                                  num_heads, head_dim, ps, max_pages, dtype, false, s);
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
    if (select(r0, n) != hipSuccess) return DSA_ERR_LAUNCH;
  }
  return DSA_OK;
}

int dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, const int32_t* row_req, const int32_t* idx,
                    int rows, int num_q_heads, int num_kv_heads, int head_dim, int k,
                    int page_size, int max_pages, float scale, int num_splits, float* part_o,
                    float* part_lse, dsa_dtype dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !row_req || !idx || !part_o || !part_lse)
    return DSA_ERR_NULL;
  if (rows < 0 || num_q_heads < 1 || num_kv_heads < 1 || k < 1 || max_pages < 1 ||
      num_splits < 1 || num_splits > k || !isfinite(scale))
    return DSA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return DSA_ERR_SHAPE;
  const int ps = pow2_shift(page_size);
  if (ps < 0) return DSA_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  if (!(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4 || G == 8 || G == 16))
    return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_BF16 && dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(part_o, 16) ||
      !aligned(part_lse, 4) || !aligned(block_table, 4) || !aligned(row_req, 4) ||
      !aligned(idx, 4))
    return DSA_ERR_ALIGN;
  if (rows == 0) return DSA_OK;
  if ((long long)rows * num_splits * num_kv_heads > INT32_MAX) return DSA_ERR_SHAPE;
  return launch_status(dsa::launch_sparse_attn(
      q, k_cache, v_cache, block_table, row_req, idx, rows, num_q_heads, num_kv_heads, head_dim,
      k, ps, max_pages, scale, num_splits, part_o, part_lse, dtype == DSA_BF16,
      static_cast<hipStream_t>(stream)));
}

int dsa_sparse_attn_merged(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* row_req, const int32_t* idx,
                           int rows, int num_q_heads, int num_kv_heads, int head_dim, int k,
                           int page_size, int max_pages, float scale, int num_splits, void* out,
                           float* out_lse, dsa_dtype dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !row_req || !idx || !out) return DSA_ERR_NULL;
  if (rows < 0 || num_q_heads < 1 || num_kv_heads < 1 || k < 1 || max_pages < 1 ||
      num_splits < 1 || num_splits > k || !isfinite(scale))
    return DSA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return DSA_ERR_SHAPE;
  const int ps = pow2_shift(page_size);
  if (ps < 0) return DSA_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  if (!(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4 || G == 8 || G == 16) ||
      !(num_splits == 1 || num_splits == 2 || num_splits == 4 || num_splits == 6 ||
        num_splits == 8))
    return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_BF16 && dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      (out_lse && !aligned(out_lse, 4)) || !aligned(block_table, 4) || !aligned(row_req, 4) ||
      !aligned(idx, 4))
    return DSA_ERR_ALIGN;
  if (rows == 0) return DSA_OK;
  if ((long long)rows * num_kv_heads > INT32_MAX) return DSA_ERR_SHAPE;
  return launch_status(dsa::launch_sparse_attn_merged(
      q, k_cache, v_cache, block_table, row_req, idx, rows, num_q_heads, num_kv_heads, head_dim,
      k, ps, max_pages, scale, num_splits, out, out_lse, dtype == DSA_BF16,
      static_cast<hipStream_t>(stream)));
}

int dsa_group_attn(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* row_req, const int32_t* idx,
                   const int32_t* groups, int num_groups, int rows, int num_q_heads,
                   int num_kv_heads, int head_dim, int k, int page_size, int max_pages,
                   float scale, void* out, float* out_lse, dsa_dtype dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !row_req || !idx || !out) return DSA_ERR_NULL;
  if (num_groups > 0 && !groups) return DSA_ERR_NULL;
  if (rows < 0 || num_groups < 0 || num_groups > rows || num_q_heads < 1 || num_kv_heads < 1 ||
      k < 1 || max_pages < 1 || !isfinite(scale))
    return DSA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return DSA_ERR_SHAPE;
  const int ps = pow2_shift(page_size);
  if (ps < 0) return DSA_ERR_SHAPE;
  if (dtype != DSA_BF16 || head_dim != 128 || num_q_heads / num_kv_heads != 8)
    return DSA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) ||
      (out_lse && !aligned(out_lse, 4)) || !aligned(block_table, 4) || !aligned(row_req, 4) ||
      !aligned(idx, 4) || (groups && !aligned(groups, 4)))
    return DSA_ERR_ALIGN;
  if ((long long)num_groups * num_kv_heads > INT32_MAX) return DSA_ERR_SHAPE;
  if (num_groups == 0) return DSA_OK;
  return launch_status(dsa::launch_group_attn(q, k_cache, v_cache, block_table, row_req, idx,
                                              groups, num_groups, num_kv_heads, k, ps, max_pages,
                                              scale, out, out_lse,
                                              static_cast<hipStream_t>(stream)));
}

int dsa_sparse_attn_merged_splits(int rows, int num_q_heads, int num_kv_heads, int head_dim,
                                  int k, dsa_dtype dtype, int* num_splits) {
  if (!num_splits) return DSA_ERR_NULL;
  if (rows < 1 || num_q_heads < 1 || num_kv_heads < 1 || k < 1 ||
      num_q_heads % num_kv_heads != 0)
    return DSA_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  if (!(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4 || G == 8 || G == 16) ||
      (dtype != DSA_BF16 && dtype != DSA_F32))
    return DSA_ERR_UNSUPPORTED;
  *num_splits = dsa::merged_default_splits(rows, num_q_heads, num_kv_heads, head_dim, k,
                                           dtype == DSA_BF16);
  return DSA_OK;
}

int dsa_sparse_attn_splits(int rows, int num_q_heads, int num_kv_heads, int head_dim, int k,
                           dsa_dtype dtype, int* num_splits) {
  if (!num_splits) return DSA_ERR_NULL;
  if (rows < 1 || num_q_heads < 1 || num_kv_heads < 1 || k < 1 ||
      num_q_heads % num_kv_heads != 0)
    return DSA_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  if (!(head_dim == 64 || head_dim == 128) || !(G == 1 || G == 2 || G == 4 || G == 8 || G == 16) ||
      (dtype != DSA_BF16 && dtype != DSA_F32))
    return DSA_ERR_UNSUPPORTED;
  *num_splits = dsa::attn_default_splits(rows, num_q_heads, num_kv_heads, head_dim, k,
                                         dtype == DSA_BF16);
  return DSA_OK;
}

int dsa_merge(const float* part_o, const float* part_lse, int rows, int num_q_heads, int head_dim,
              int num_splits, void* out, float* out_lse, dsa_dtype out_dtype, void* stream) {
  if (!part_o || !part_lse || !out) return DSA_ERR_NULL;
  if (rows < 0 || num_q_heads < 1 || head_dim < 1 || head_dim > 256 || num_splits < 1)
    return DSA_ERR_SHAPE;
  if (out_dtype != DSA_BF16 && out_dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  if (!aligned(part_o, 16) || !aligned(out, 16) || !aligned(part_lse, 4) ||
      (out_lse && !aligned(out_lse, 4)))
    return DSA_ERR_ALIGN;
  if (rows == 0) return DSA_OK;
  if ((long long)rows * num_q_heads > INT32_MAX - 4) return DSA_ERR_SHAPE;
  return launch_status(dsa::launch_merge(part_o, part_lse, rows, num_q_heads, head_dim,
                                         num_splits, out, out_lse, out_dtype == DSA_BF16,
                                         static_cast<hipStream_t>(stream)));
}

int dsa_read_probe(const void* src, long long bytes, float* sink, int sink_len, void* stream) {
  if (!src || !sink) return DSA_ERR_NULL;
  if (bytes < 16 || (bytes & 15) != 0 || sink_len < 1) return DSA_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return DSA_ERR_ALIGN;
  int cus = dsa::device_cus();
  if (cus <= 0) cus = 256;
  const int blocks = sink_len < 8 * cus ? sink_len : 8 * cus;
  return launch_status(
      dsa::launch_read_probe(src, bytes, sink, blocks, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
