// Internal launcher interface between the C ABI (dsa_api.cpp) and the HIP
// kernels. Arguments are validated by the caller; every launcher enqueues on
// `stream` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <mutex>
#include <stdint.h>

namespace dsa {

// Workgroups of `kernel` (launched with `block` threads) that the current
// device runs at once: compute units x resident workgroups per unit. 0 on a
// HIP error. Looked up once per (device, kernel, block) and kept.
int device_capacity(const void* kernel, int block);
// Compute units of the current device (looked up once per device); 0 on a
// HIP error.
int device_cus();

// A second stream of the current device (non-blocking, default priority) with
// a fork and a join event, made once and kept: a launcher records `fork` on
// its stream, has this stream wait for it, enqueues independent work here,
// records `join` and has its own stream wait for that -- all while holding
// `lock`, so that launchers on several host threads never wait on each
// other's event records. Null on a HIP error.
struct SideStream {
  hipStream_t stream;
  hipEvent_t fork, join;
  std::mutex* lock;
};
SideStream* side_stream();

// Keys a workgroup of the bf16 indexer covers for one row (a multiple of 64):
// the chunks of all blocks fill the device about once, at most 2048 keys.
int indexer_chunk_keys(int num_blocks, int width, int num_heads, int head_dim, bool full);

// Splits of the k slots that fill the device with attention waves about once.
int attn_default_splits(int rows, int hq, int hkv, int d, int k, bool bf16);

// Whether launch_indexer_bf16 scores the blocks of several rows with the
// block kernel (query blocks in registers, keys shared through LDS); blocks
// of one row then go to the row kernel, launched after it.
bool indexer_uses_blocks(int rows, int num_blocks);
// Keys a workgroup of the block kernel covers (a multiple of 128, at most 8192).
int indexer_block_chunk_keys(int num_blocks, int width, int num_heads, int head_dim, bool full);

hipError_t launch_indexer_bf16(const void* q_idx, const float* w, const void* kcache,
                               const int32_t* bt, const int32_t* row_req, const int32_t* row_len,
                               const int32_t* blocks, int num_blocks, int rows, float* scores,
                               int width, int num_heads, int head_dim, int page_shift,
                               int max_pages, bool full, int score_row0, hipStream_t stream,
                               uint32_t* hist = nullptr, long long total_keys = 0);

hipError_t launch_indexer_f32(const float* q_idx, const float* w, const float* kcache,
                              const int32_t* bt, const int32_t* row_req, const int32_t* row_len,
                              const int32_t* blocks, int num_blocks, float* scores, int width,
                              int num_heads, int head_dim, int page_shift, int max_pages,
                              int score_row0, hipStream_t stream);

// total_keys: the sum of the row lengths if the host knows it, else 0.
hipError_t launch_topk(const float* scores, const int32_t* row_len, int rows, int width, int k,
                       int32_t* idx, hipStream_t stream, long long total_keys = 0);
// Segments of `seg` positions per row of `width` (the stage-1 workgroups per row).
int topk_segments(int width, int seg);
// Segment length for dsa_topk_chunked when it beats the one-pass kernel, else 0.
int topk_suggest_chunk(int rows, int width, int k, bool full);
// Two-stage exact top-k: per-segment winners into cand [rows][nseg][k], then
// each row's top-k over them into idx. Requires seg >= k.
hipError_t launch_topk_chunked(const float* scores, const int32_t* row_len, int rows, int width,
                               int k, int seg, int32_t* cand, int32_t* idx, hipStream_t stream);

// Histogram-driven exact top-k: hist [rows][4096] counts each row's scores
// by the top 12 bits of their order keys (as the indexer leaves it); the
// selection equals launch_topk's and hist is left cleared.
hipError_t launch_topk_hist(const float* scores, const int32_t* row_len, uint32_t* hist, int rows,
                            int width, int k, int32_t* idx, hipStream_t stream,
                            long long total_keys = 0);
// Adds each row's score counts to hist [rows][4096] (cleared first when
// `clear`), from the scores already written.
hipError_t launch_score_hist(const float* scores, const int32_t* row_len, int rows, int width,
                             uint32_t* hist, bool clear, hipStream_t stream);

hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* bt,
                              const int32_t* row_req, const int32_t* idx, int rows, int hq,
                              int hkv, int d, int k, int page_shift, int max_pages, float scale,
                              int num_splits, float* part_o, float* part_lse, bool bf16,
                              hipStream_t stream);

hipError_t launch_sparse_attn_merged(const void* q, const void* kc, const void* vc,
                                     const int32_t* bt, const int32_t* row_req, const int32_t* idx,
                                     int rows, int hq, int hkv, int d, int k, int page_shift,
                                     int max_pages, float scale, int num_splits, void* out,
                                     float* out_lse, bool bf16, hipStream_t stream);

// Prefill group attention (bf16, head dim 128, 8 query heads per KV head):
// each group {first_row, n_rows <= 8} of rows of one request attends the
// union of its rows' ascending selections, row r only its own keys; writes
// out / out_lse of the groups' rows.
hipError_t launch_group_attn(const void* q, const void* kc, const void* vc, const int32_t* bt,
                             const int32_t* row_req, const int32_t* idx, const int32_t* groups,
                             int num_groups, int hkv, int k, int page_shift, int max_pages,
                             float scale, void* out, float* out_lse, hipStream_t stream);

// Split count for the merged variant: attn_default_splits rounded down to 1/2/4/8.
int merged_default_splits(int rows, int hq, int hkv, int d, int k, bool bf16);

hipError_t launch_merge(const float* part_o, const float* part_lse, int rows, int hq, int d,
                        int num_splits, void* out, float* out_lse, bool out_bf16,
                        hipStream_t stream);

// Workgroup id -> work item such that the items each XCD runs form one
// contiguous range. Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup i runs on XCD i % 8); item ranges that share data (the key
// chunks of one row, the rows of one request) then share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int wg, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = wg & 7, j = wg >> 3;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// Streaming-read probe (benchmark floor): per-workgroup sums into sink[blocks].
hipError_t launch_read_probe(const void* src, long long bytes, float* sink, int blocks,
                             hipStream_t stream);

}  // namespace dsa
