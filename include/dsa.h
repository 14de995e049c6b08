/*
 * dsa.h -- C ABI of libdsa.so, the MI355X (gfx950) paged DeepSeek-sparse-
 * attention step:
 *
 *   indexer scores -> length-bounded exact top-k -> GQA sparse attention
 *   split over the k slots -> log-sum-exp merge
 *
 * The method is the one of Megatron-LM pull request 7211 ("native dynamic
 * inference for simplified DSA over GQA"); each entry point names the commit
 * of that pull request whose message defines its operation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" are HIP device memory, dense row-major, owned by
 *   the caller; the library never allocates, frees, synchronizes, or reads
 *   device memory on the host. Pointers marked "host" are host memory.
 * - "stream" is a hipStream_t (NULL = the default stream). All work is
 *   enqueued on it in call order; the calls return before the work finishes.
 * - Return value: DSA_OK (0) or a negative dsa_status. Every host-visible
 *   argument is checked before anything is enqueued; on a negative status
 *   nothing was launched and no output was written. DSA_ERR_LAUNCH reports a
 *   failed kernel launch.
 * - Device-resident metadata (block-table entries, row lengths, selected
 *   positions, score blocks) is a caller contract and is not read on the
 *   host: block_table[q][j] must name a valid page for every page a row of
 *   request q reaches, row_len[r] must not exceed the score width or the
 *   request's cached tokens, and every selected position must be -1 or lie in
 *   [0, row_len[r]). Violations are undefined behaviour.
 * - Per-step integers (rows, width, k, lengths, number of splits) are runtime
 *   values, so the launch shape depends only on the call's arguments and the
 *   kernels can be replayed with new lengths in the same buffers (commit
 *   "Treat every query token of a step ... as a row": launch sizes depend only
 *   on the padded batch; the PR description: graph replay with changing token
 *   positions and active lengths).
 * - The calls are thread-safe: the library keeps no mutable global state,
 *   except the fixed per-device workspace of dsa_topk_chunked_noalloc (and
 *   its device address, looked up once per device), whose calls must not
 *   overlap on one device.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_F32 = 0,  /* IEEE float32 */
  DSA_BF16 = 1  /* bfloat16 (upper half of a float32) */
} dsa_dtype;

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  DSA_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned */
  DSA_ERR_UNSUPPORTED = -4, /* head count / head dim / dtype combination not built */
  DSA_ERR_WORKSPACE = -5,   /* a workspace buffer is too small */
  DSA_ERR_LAUNCH = -6       /* the kernel launch failed */
} dsa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* dsa_status_string(int status);

/* Version of this ABI (incremented on incompatible change). */
int dsa_abi_version(void);

/* ------------------------------------------------------------------------
 * Row plan (host only; no HIP call)
 *
 * Commit "Treat every query token of a step, decode or prefill, as a row that
 * routes to the top-k of its causal prefix": the rows of a step, and its
 * score blocks (consecutive rows of one request scored against shared key
 * tiles).
 * ------------------------------------------------------------------------ */

/*
 * dsa_plan_rows: request q has prior[q] >= 0 tokens cached before the step
 * and appends new_tokens[q] >= 0 tokens (1 = decode). Each new token is a
 * row, request by request, in token order: row_req = q and row_len =
 * prior[q] + i + 1 for its i-th new token (a row attends positions
 * [0, row_len)). Writes *num_rows = sum(new_tokens) and the first *num_rows
 * entries of row_req / row_len (host int32 arrays of max_rows entries).
 * Errors: NULL pointer; num_reqs < 0, a negative count, a length that
 * overflows int32, or more rows than max_rows -> DSA_ERR_SHAPE.
 */
int dsa_plan_rows(int num_reqs, const int32_t* prior, const int32_t* new_tokens, int max_rows,
                  int32_t* row_req, int32_t* row_len, int* num_rows);

/*
 * dsa_plan_blocks: splits rows into score blocks, runs of at most
 * max_rows_per_block consecutive rows with equal row_req. Writes
 * (first_row, n_rows) pairs to blocks (host int32 [max_blocks][2]) and their
 * count to *num_blocks. Errors: NULL pointer; rows < 0; max_rows_per_block
 * < 1; more blocks than max_blocks -> DSA_ERR_SHAPE.
 */
int dsa_plan_blocks(int rows, const int32_t* row_req, int max_rows_per_block, int max_blocks,
                    int32_t* blocks, int* num_blocks);

/*
 * dsa_score_width: the score buffer's row stride for these rows: the largest
 * row_len rounded up to a multiple of 64 (at least 64). row_len is host
 * memory. Errors: NULL pointer, rows < 0, a negative length.
 */
int dsa_score_width(int rows, const int32_t* row_len, int* width);

/* ------------------------------------------------------------------------
 * dsa_indexer_scores -- lightning-indexer scores.
 *
 * Commit "Replace the CuTe decode kernels with two Triton kernels": the
 * indexer streams page-contiguous key tiles on the matrix cores, and each
 * row is scored only up to its length. For row r of request q = row_req[r]
 * and every position s < row_len[r]:
 *
 *   scores[r][s] = sum_h w[r][h] * max(0, sum_j q_idx[r][h][j] * kI[q][s][j])
 *
 * where kI[q][s] = k_idx_cache[block_table[q][s / page_size]][s % page_size].
 * Positions [row_len[r], width) of the row are not written. -0.0 is written as
 * +0.0. bf16 inputs are multiplied exactly and accumulated in fp32 on MFMA;
 * fp32 inputs use fp32 FMA.
 *
 *   q_idx        device [rows][num_heads][head_dim]    dtype
 *   w            device [rows][num_heads]               float32
 *   k_idx_cache  device [num_pages][page_size][head_dim] dtype
 *   block_table  device [num_reqs][max_pages]           int32
 *   row_req      device [rows]                          int32
 *   row_len      device [rows]                          int32
 *   blocks       device [num_blocks][2] (first_row, n_rows) int32, or NULL
 *                for one row per block; rows of a block are consecutive and
 *                share a request (dsa_plan_blocks' plan): a block of several
 *                rows is scored against its first row's block-table row, with
 *                each key tile read once for all of its rows
 *   scores       device [rows][width]                   float32 (output)
 *
 * Supported: bf16 with head_dim in {64, 128}, num_heads in {32, 64} and
 * page_size >= 16; fp32 with head_dim in {32, 64, 128} and 1 <= num_heads
 * <= 64. page_size is a power of two; width is a positive multiple of 4; q_idx,
 * k_idx_cache and scores are 16-byte aligned.
 * ------------------------------------------------------------------------ */
int dsa_indexer_scores(const void* q_idx, const float* w, const void* k_idx_cache,
                       const int32_t* block_table, const int32_t* row_req, const int32_t* row_len,
                       const int32_t* blocks, int num_blocks, float* scores, int rows, int width,
                       int num_heads, int head_dim, int page_size, int max_pages, dsa_dtype dtype,
                       void* stream);

/* dsa_indexer_scores with a scheduling hint: total_keys = the sum of row_len
 * over the rows (known on the host from the row plan; 0 = unknown). Rows that
 * fill at least 90% of rows x width are scored in larger key chunks (no
 * ragged tail to balance); a ragged batch of at most 256 rows in one-row
 * blocks spreads the key chunks its rows actually hold evenly over the
 * XCDs, with the grid sized from the hint (a hint below the true sum only
 * makes workgroups take several chunks). The scores are identical either
 * way; the launch shape depends only on the arguments, so a replayed step
 * must pass the same hint. total_keys outside [0, rows * width]:
 * DSA_ERR_SHAPE. */
int dsa_indexer_scores_total(const void* q_idx, const float* w, const void* k_idx_cache,
                             const int32_t* block_table, const int32_t* row_req,
                             const int32_t* row_len, const int32_t* blocks, int num_blocks,
                             float* scores, int rows, int width, int num_heads, int head_dim,
                             int page_size, int max_pages, dsa_dtype dtype, long long total_keys,
                             void* stream);

/* ------------------------------------------------------------------------
 * Score histograms for the selection's threshold.
 *
 * Commit "When a step's context bound reaches 64K keys, each row now
 * thresholds at a sampled score ...": each row gets a threshold, a filter
 * keeps the keys reaching it, and the exact top k is taken among those
 * candidates. Here the threshold is exact: the histogram of a row's scores
 * over the top 12 bits of their order keys, where the order key of a float32
 * score x (-0.0 taken as +0.0) is bits(x) ^ 0xFFFFFFFF for x < 0 and
 * bits(x) | 0x80000000 otherwise (unsigned order of keys = order of scores),
 * and
 *
 *   hist[r][b] = #{ s < row_len[r] : order_key(scores[r][s]) >> 20 == b },
 *
 * b in [0, 4096). The bin where the count from the top first reaches k holds
 * the k-th largest score, so every key of a higher bin is selected and only
 * that bin's keys need ranking.
 * ------------------------------------------------------------------------ */

/* dsa_indexer_scores_total that also adds each row's score histogram to
 * hist (device uint32 [rows][4096], 16-byte aligned), which must be all zero
 * on entry -- as dsa_topk_hist leaves it (allocate it zeroed once). Decode
 * batches count their scores inside the scoring kernel; rows of multi-row
 * score blocks and fp32 inputs are counted by one more launch over the
 * written scores. Errors as dsa_indexer_scores_total; NULL hist:
 * DSA_ERR_NULL. */
int dsa_indexer_scores_hist(const void* q_idx, const float* w, const void* k_idx_cache,
                            const int32_t* block_table, const int32_t* row_req,
                            const int32_t* row_len, const int32_t* blocks, int num_blocks,
                            float* scores, uint32_t* hist, int rows, int width, int num_heads,
                            int head_dim, int page_size, int max_pages, dsa_dtype dtype,
                            long long total_keys, void* stream);

/* dsa_score_hist: writes the histogram above of the scores already in
 * scores (device float32 [rows][width]) to hist (device uint32
 * [rows][4096], 16-byte aligned; cleared first, then counted). */
int dsa_score_hist(const float* scores, const int32_t* row_len, int rows, int width,
                   uint32_t* hist, void* stream);

/* ------------------------------------------------------------------------
 * dsa_topk -- length-bounded exact top-k.
 *
 * Commits "Replace the CuTe decode kernels with two Triton kernels" (the
 * selection reads each row only up to its length), "When a step's context
 * bound reaches 64K keys ..." (the result is the exact top k), and "Replace
 * the Triton radix selector with torch.topk ..." (valid negative-infinity
 * scores rank ahead of padding). For every row r with L = row_len[r]:
 * selects the min(k, L) positions of [0, L) with the largest scores, ties to
 * the lower position, -0.0 equal to +0.0, and writes them to idx[r] in
 * ascending position order, followed by -1 in the remaining slots.
 * NaN scores are outside the contract (never out-of-bounds, result
 * unspecified).
 *
 *   scores   device [rows][width] float32, 16-byte aligned
 *   row_len  device [rows] int32
 *   idx      device [rows][k] int32 (output)
 *
 * 1 <= k <= width; width a positive multiple of 4.
 * ------------------------------------------------------------------------ */
int dsa_topk(const float* scores, const int32_t* row_len, int rows, int width, int k,
             int32_t* idx, void* stream);

/* dsa_topk with a scheduling hint: total_keys = the sum of row_len over the
 * rows (known on the host from the row plan; 0 = unknown). Batches of many
 * rows that are short on average run in smaller workgroups. The indices are
 * identical either way; the launch shape depends only on the arguments, so a
 * replayed step must pass the same hint. total_keys outside
 * [0, rows * width]: DSA_ERR_SHAPE. */
int dsa_topk_total(const float* scores, const int32_t* row_len, int rows, int width, int k,
                   long long total_keys, int32_t* idx, void* stream);

/* dsa_topk from the rows' score histograms (dsa_indexer_scores_hist or
 * dsa_score_hist for these scores): the threshold bin comes from hist, the
 * keys at or above it are compacted in position order into on-chip memory
 * (after further radix passes over the row while they would not fit), and
 * the selection is finished among them -- a long row is read once or twice
 * instead of once per radix pass. The indices equal dsa_topk's bit for bit;
 * hist is left all zero for the next step. A histogram that does not count
 * the row's row_len scores makes the row ranked from scratch (still exact).
 *
 *   hist  device uint32 [rows][4096], 16-byte aligned (read, then cleared)
 *   total_keys  as for dsa_topk_total
 *
 * Errors as dsa_topk_total; NULL hist: DSA_ERR_NULL. */
int dsa_topk_hist(const float* scores, const int32_t* row_len, uint32_t* hist, int rows,
                  int width, int k, long long total_keys, int32_t* idx, void* stream);

/* ------------------------------------------------------------------------
 * dsa_topk_chunked -- the same selection as dsa_topk, in two stages.
 *
 * Commit "Replace handwritten inline PTX selection with a CuTe DSL histogram
 * fast path ..." keeps exact chunk merging for long contexts. Stage 1 takes
 * the exact top-k of every segment [c*chunk, (c+1)*chunk) of every row (one
 * workgroup per segment, so a long row spreads over many compute units);
 * stage 2 takes each row's exact top-k among its segments' winners. Every
 * position of the row's top-k is among its segment's top-k, so the result is
 * dsa_topk's, bit for bit: same positions, same order, same -1 padding.
 *
 *   scores   device [rows][width] float32, 16-byte aligned
 *   row_len  device [rows] int32
 *   cand     device int32 workspace of cand_slots entries, at least
 *            2 * rows * ceil(width / chunk) * k (dsa_topk_chunked_slots):
 *            the segment winners' positions, then their sort keys;
 *            overwritten, holds no result
 *   idx      device [rows][k] int32 (output)
 *
 * k <= chunk <= 2^20, chunk a multiple of 4; 1 <= k <= width; width a
 * positive multiple of 4. cand_slots too small: DSA_ERR_WORKSPACE.
 * ------------------------------------------------------------------------ */
int dsa_topk_chunked(const float* scores, const int32_t* row_len, int rows, int width, int k,
                     int chunk, int32_t* cand, long long cand_slots, int32_t* idx, void* stream);

/* Candidate slots dsa_topk_chunked needs for these sizes (host). */
int dsa_topk_chunked_slots(int rows, int width, int k, int chunk, long long* slots);

/* ------------------------------------------------------------------------
 * dsa_topk_chunked_noalloc -- dsa_topk_chunked without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same selection and result as dsa_topk_chunked, bit for bit. The candidate
 * workspace is a fixed array inside the library, DSA_TOPK_NOALLOC_MAX_SLOTS
 * int32 slots (16 MiB) on each device the library runs on, held until the
 * process ends; the call allocates and frees nothing. Every call on a device
 * shares that device's array and leaves its contents behind (nothing in it
 * needs clearing: stage 1 writes every entry stage 2 reads). Calls that
 * overlap on one device -- on two streams, or from two host threads without
 * ordering -- race on the array and give undefined results.
 *
 *   scores, row_len, idx, k, chunk: as for dsa_topk_chunked
 *
 * Sizes needing more than DSA_TOPK_NOALLOC_MAX_SLOTS candidate slots
 * (dsa_topk_chunked_slots; e.g. 64 rows of 204800 positions with k = 2048 and
 * chunk = 32768 need 1835008) return DSA_ERR_WORKSPACE before any launch;
 * other errors as for dsa_topk_chunked; DSA_ERR_LAUNCH also when the array's
 * device address cannot be found on the current device.
 * ------------------------------------------------------------------------ */
#define DSA_TOPK_NOALLOC_MAX_SLOTS (1LL << 22)
int dsa_topk_chunked_noalloc(const float* scores, const int32_t* row_len, int rows, int width,
                             int k, int chunk, int32_t* idx, void* stream);

/* The segment length at which dsa_topk_chunked is expected to beat dsa_topk
 * on the current device for these sizes, or 0 (host): rows longer than one
 * workgroup holds in registers, and either rows that fill the width
 * (total_keys, the sum of the row lengths, >= 90% of rows * width) or few
 * enough segments to run at once. total_keys outside [0, rows * width]:
 * DSA_ERR_SHAPE. */
int dsa_topk_chunk_suggest(int rows, int width, int k, long long total_keys, int* chunk);

/* ------------------------------------------------------------------------
 * dsa_indexer_topk_windowed -- indexer scores and top-k in row windows.
 *
 * Commit "Score and select rows in windows whose score buffer fits ...": the
 * rows are scored and selected a window at a time through one caller-given
 * score buffer, so its size bounds the score memory at any context length.
 * A window holds at most window_rows = score_buffer_bytes / (width * 4) rows
 * (dsa_select_window_rows); with score blocks it is a run of whole blocks.
 * The window count depends only on the sizes and the block plan, so the
 * launch sequence is the same for every step of those sizes. Each window
 * runs the indexer on its rows into the buffer, then dsa_topk
 * (topk_chunk == 0) or dsa_topk_chunked (topk_chunk > 0, with cand sized for
 * one window) into those rows of idx. Results equal those of
 * dsa_indexer_scores over all rows followed by the same selection.
 *
 *   q_idx, w, k_idx_cache, block_table, row_req, row_len: as for
 *            dsa_indexer_scores (all rows)
 *   blocks_host, blocks_dev, num_blocks: optional score blocks (the
 *            dsa_plan_blocks plan, on the host and a device copy of it), or
 *            0 and NULL for none; the plan must cover the rows in order, and
 *            a block longer than a window returns DSA_ERR_WORKSPACE
 *   score_buffer  device float32 workspace of score_buffer_bytes, 16-byte
 *            aligned; overwritten, holds no result
 *   cand, cand_slots  as for dsa_topk_chunked, for window_rows rows (unused,
 *            may be NULL, when topk_chunk == 0)
 *   idx      device [rows][k] int32 (output)
 *
 * A buffer smaller than one score row: DSA_ERR_WORKSPACE.
 * ------------------------------------------------------------------------ */
int dsa_indexer_topk_windowed(const void* q_idx, const float* w, const void* k_idx_cache,
                              const int32_t* block_table, const int32_t* row_req,
                              const int32_t* row_len, const int32_t* blocks_host,
                              const int32_t* blocks_dev, int num_blocks, int rows, int width,
                              int num_heads, int head_dim, int page_size, int max_pages,
                              dsa_dtype dtype, int k, float* score_buffer,
                              long long score_buffer_bytes, int topk_chunk, int32_t* cand,
                              long long cand_slots, int32_t* idx, void* stream);

/* Rows per window for a score buffer of score_buffer_bytes (host). */
int dsa_select_window_rows(int width, long long score_buffer_bytes, int* window_rows);

/* ------------------------------------------------------------------------
 * dsa_sparse_attn -- GQA sparse attention over split k-slot slices.
 *
 * Commit "Replace the CuTe decode kernels with two Triton kernels": one
 * program serves all query heads of a KV group, reading each selected key and
 * value once, and the top-k slots are split across programs; commit "Restore
 * the upstream Blackwell FP32 probability reduction": probabilities stay fp32
 * through the value reduction. Split s covers slots [s*c, min(k, (s+1)*c))
 * with c = ceil(k / num_splits). For row r, query head h, KV head
 * g = h / (num_q_heads / num_kv_heads), and the valid selected positions p_j
 * (idx >= 0) of the split:
 *
 *   z_j = scale * q[r][h] . K[p_j][g],  m = max_j z_j,  l = sum_j exp(z_j - m)
 *   part_o[r][h][s]   = sum_j exp(z_j - m) V[p_j][g] / l
 *   part_lse[r][h][s] = m + ln l            (0 and -inf for an empty split)
 *
 * with K[p] = k_cache[block_table[q][p / page_size]][p % page_size] for the
 * row's request q (V likewise).
 *
 *   q        device [rows][num_q_heads][head_dim]                 dtype
 *   k_cache  device [num_pages][page_size][num_kv_heads][head_dim] dtype
 *   v_cache  device, same layout as k_cache
 *   block_table, row_req: as for dsa_indexer_scores
 *   idx      device [rows][k] int32 (dsa_topk's output)
 *   part_o   device [rows][num_q_heads][num_splits][head_dim] float32 (output)
 *   part_lse device [rows][num_q_heads][num_splits] float32 (output)
 *
 * Supported: head_dim in {64, 128}; num_q_heads / num_kv_heads in
 * {1, 2, 4, 8, 16}; 1 <= num_splits <= k; page_size a power of two; q,
 * k_cache, v_cache and part_o 16-byte aligned.
 * ------------------------------------------------------------------------ */
int dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, const int32_t* row_req, const int32_t* idx,
                    int rows, int num_q_heads, int num_kv_heads, int head_dim, int k,
                    int page_size, int max_pages, float scale, int num_splits, float* part_o,
                    float* part_lse, dsa_dtype dtype, void* stream);

/*
 * dsa_sparse_attn_splits: a num_splits for dsa_sparse_attn with these shapes
 * on the current HIP device -- enough splits that one launch has about two
 * thirds as many waves as the device runs at once (more splits add partial
 * traffic and per-wave setup, fewer leave compute units idle), each split
 * keeping at least 32 slots.
 * Queries the device (compute-unit count, kernel occupancy); allocates
 * nothing. Errors: NULL pointer; rows, k or head counts < 1 or
 * num_q_heads % num_kv_heads != 0 -> DSA_ERR_SHAPE; an unsupported
 * head_dim / group size / dtype -> DSA_ERR_UNSUPPORTED.
 */
int dsa_sparse_attn_splits(int rows, int num_q_heads, int num_kv_heads, int head_dim, int k,
                           dsa_dtype dtype, int* num_splits);

/* ------------------------------------------------------------------------
 * dsa_sparse_attn_merged -- dsa_sparse_attn followed by dsa_merge in one
 * launch (same commits). The num_splits splits of a (row, KV group) run in
 * one workgroup and are merged on chip; the split partials never reach
 * device memory. out / out_lse equal, bit for bit, what dsa_sparse_attn with
 * the same num_splits followed by dsa_merge writes.
 *
 *   q, k_cache, v_cache, block_table, row_req, idx: as for dsa_sparse_attn
 *   out      device [rows][num_q_heads][head_dim] dtype (bf16 rounds to
 *            nearest even) (output)
 *   out_lse  device [rows][num_q_heads] float32 (output), or NULL
 *
 * Supported: as dsa_sparse_attn, with num_splits in {1, 2, 4, 6, 8} and
 * num_splits <= k; out 16-byte aligned. (Six splits of any shape, and four
 * or eight splits of bf16 rows with head_dim 128 and eight query heads per
 * KV group, run two pairs per workgroup; the result does not depend on it.)
 * ------------------------------------------------------------------------ */
int dsa_sparse_attn_merged(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* row_req, const int32_t* idx,
                           int rows, int num_q_heads, int num_kv_heads, int head_dim, int k,
                           int page_size, int max_pages, float scale, int num_splits, void* out,
                           float* out_lse, dsa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * dsa_group_attn -- prefill group attention over the union of selections.
 *
 * Commit "--dsa-inference-backend flashinfer ...": prefill tiles attend each
 * 8-token group over the union of the keys its tokens selected, with a
 * per-token bitmask; commit "Restore the upstream Blackwell FP32 probability
 * reduction": probabilities stay fp32 through the value reduction. For every
 * group g = {first_row, n_rows} (groups[g][0], groups[g][1]; 1 <= n_rows <= 8
 * consecutive rows of one request, scored against first_row's block-table
 * row) and each of its rows r, writes what dsa_sparse_attn with one split
 * followed by dsa_merge writes for row r (up to rounding order):
 *
 *   out[r][h] = sum_j softmax_j(scale * q[r][h] . K[p_j][g]) V[p_j][g],
 *   out_lse[r][h] = the log-sum-exp,
 *
 * over row r's valid selections p_j. The keys of the union are read once per
 * group and KV head, and its 64 query rows (8 rows x 8 heads) run on the
 * matrix cores; the fp32 probabilities enter the value product as three exact
 * bf16 terms. Each row's valid selections must be distinct and ascending,
 * followed by -1 padding (dsa_topk's output); rows not in any group are not
 * written.
 *
 *   q, k_cache, v_cache, block_table, row_req, idx: as for dsa_sparse_attn
 *   groups   device int32 [num_groups][2]: (first_row, n_rows), rows in
 *            [0, rows) (a caller contract, like the score blocks)
 *   out      device [rows][num_q_heads][128] bf16 (output, the groups' rows)
 *   out_lse  device [rows][num_q_heads] float32 (output), or NULL
 *
 * Supported: bf16, head_dim 128, num_q_heads / num_kv_heads = 8; page_size a
 * power of two; q, k_cache, v_cache 16-byte aligned. Otherwise
 * DSA_ERR_UNSUPPORTED / DSA_ERR_SHAPE / DSA_ERR_ALIGN as for dsa_sparse_attn.
 * ------------------------------------------------------------------------ */
int dsa_group_attn(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* row_req, const int32_t* idx,
                   const int32_t* groups, int num_groups, int rows, int num_q_heads,
                   int num_kv_heads, int head_dim, int k, int page_size, int max_pages,
                   float scale, void* out, float* out_lse, dsa_dtype dtype, void* stream);

/* dsa_sparse_attn_merged_splits: a num_splits for dsa_sparse_attn_merged
 * with these shapes on the current device. bf16 rows with head_dim 128 and
 * eight query heads per KV group (the matrix-core kernel): the smallest of
 * 1, 2, 4, 8 that puts about seven waves (rows x KV groups x splits) on
 * every compute unit, at most k / 16. Other shapes: 6 when rows x KV groups
 * x 6 waves fill the device in about one round, else dsa_sparse_attn_splits
 * rounded down to 1, 2, 4 or 8. Errors as for dsa_sparse_attn_splits. */
int dsa_sparse_attn_merged_splits(int rows, int num_q_heads, int num_kv_heads, int head_dim,
                                  int k, dsa_dtype dtype, int* num_splits);

/* ------------------------------------------------------------------------
 * dsa_merge -- log-sum-exp merge of the split partials (flash decoding,
 * commit "Replace the CuTe decode kernels with two Triton kernels").
 * For each row r and head h, over the splits s:
 *
 *   M = max_s lse_s,  W = sum_s exp(lse_s - M),
 *   out[r][h] = sum_s exp(lse_s - M) o_s / W,  out_lse[r][h] = M + ln W
 *
 * and out = 0, out_lse = -inf when every split is empty. Up to 8 splits are
 * summed in split order (the order dsa_sparse_attn_merged uses); more splits
 * are summed as four interleaved partial merges, rescaled and added.
 *
 *   part_o, part_lse  device, as written by dsa_sparse_attn
 *   out      device [rows][num_q_heads][head_dim] out_dtype (bf16 rounds to
 *            nearest even) (output)
 *   out_lse  device [rows][num_q_heads] float32 (output), or NULL
 *
 * 1 <= head_dim <= 256; num_splits >= 1; part_o and out 16-byte aligned.
 * ------------------------------------------------------------------------ */
int dsa_merge(const float* part_o, const float* part_lse, int rows, int num_q_heads, int head_dim,
              int num_splits, void* out, float* out_lse, dsa_dtype out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * dsa_read_probe -- streaming-read probe (not part of the step).
 *
 * Reads `bytes` of `src` once with 16-byte loads and writes per-workgroup
 * fp32 sums to sink[0 .. min(sink_len, 8 * CUs)); its duration gives the
 * device's practical read bandwidth, the floor the step's bandwidth-bound
 * kernels are compared with.
 *
 *   src   device, 16-byte aligned; bytes a positive multiple of 16
 *   sink  device float32 [sink_len] (output)
 * ------------------------------------------------------------------------ */
int dsa_read_probe(const void* src, long long bytes, float* sink, int sink_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
