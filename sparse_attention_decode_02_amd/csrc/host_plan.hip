// Host-only entry points of libdsa.so: status strings, the ABI version, the
// row plan (commit "Treat every query token of a step ... as a row": rows
// are (request, causal length) pairs, score blocks group consecutive rows of
// one request), the score width, and the window size of the row-window path
// (commit "Score and select rows in windows ..."). Plain C++ with no HIP
// calls, so the same file also builds with a host compiler under the address
// and undefined-behaviour sanitizers (tests/test_host_sanitize.py). Every
// check runs before any output is written.

#include <limits.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace {
constexpr int kAbiVersion = 1;
}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case DSA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case DSA_ERR_UNSUPPORTED: return "head count / head dim / dtype combination not supported";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int dsa_abi_version(void) { return kAbiVersion; }

int dsa_plan_rows(int num_reqs, const int32_t* prior, const int32_t* new_tokens, int max_rows,
                  int32_t* row_req, int32_t* row_len, int* num_rows) {
  if (!num_rows || (num_reqs > 0 && (!prior || !new_tokens))) return DSA_ERR_NULL;
  if (num_reqs < 0 || max_rows < 0) return DSA_ERR_SHAPE;
  long long total = 0;
  for (int q = 0; q < num_reqs; ++q) {
    if (prior[q] < 0 || new_tokens[q] < 0) return DSA_ERR_SHAPE;
    if ((long long)prior[q] + new_tokens[q] > INT32_MAX) return DSA_ERR_SHAPE;
    total += new_tokens[q];
  }
  if (total > max_rows) return DSA_ERR_SHAPE;
  if (total > 0 && (!row_req || !row_len)) return DSA_ERR_NULL;
  int r = 0;
  for (int q = 0; q < num_reqs; ++q)
    for (int i = 0; i < new_tokens[q]; ++i, ++r) {
      row_req[r] = q;
      row_len[r] = prior[q] + i + 1;
    }
  *num_rows = r;
  return DSA_OK;
}

int dsa_plan_blocks(int rows, const int32_t* row_req, int max_rows_per_block, int max_blocks,
                    int32_t* blocks, int* num_blocks) {
  if (!num_blocks || (rows > 0 && (!row_req || !blocks))) return DSA_ERR_NULL;
  if (rows < 0 || max_rows_per_block < 1 || max_blocks < 0) return DSA_ERR_SHAPE;
  // Count first, so that a block list too long for max_blocks writes nothing.
  auto block_end = [&](int r) {
    int e = r + 1;
    while (e < rows && row_req[e] == row_req[r] && e - r < max_rows_per_block) ++e;
    return e;
  };
  int nb = 0;
  for (int r = 0; r < rows; r = block_end(r)) ++nb;
  if (nb > max_blocks) return DSA_ERR_SHAPE;
  nb = 0;
  for (int r = 0; r < rows;) {
    const int e = block_end(r);
    blocks[2 * nb] = r;
    blocks[2 * nb + 1] = e - r;
    ++nb;
    r = e;
  }
  *num_blocks = nb;
  return DSA_OK;
}

int dsa_score_width(int rows, const int32_t* row_len, int* width) {
  if (!width || (rows > 0 && !row_len)) return DSA_ERR_NULL;
  if (rows < 0) return DSA_ERR_SHAPE;
  int mx = 0;
  for (int r = 0; r < rows; ++r) {
    if (row_len[r] < 0) return DSA_ERR_SHAPE;
    if (row_len[r] > mx) mx = row_len[r];
  }
  if (mx > INT32_MAX - 63) return DSA_ERR_SHAPE;
  const int w = ((mx + 63) / 64) * 64;
  *width = w < 64 ? 64 : w;
  return DSA_OK;
}

int dsa_select_window_rows(int width, long long score_buffer_bytes, int* window_rows) {
  if (!window_rows) return DSA_ERR_NULL;
  if (width < 1 || score_buffer_bytes < 0) return DSA_ERR_SHAPE;
  const long long w = score_buffer_bytes / ((long long)width * 4);
  if (w < 1) return DSA_ERR_WORKSPACE;
  *window_rows = w > INT32_MAX ? INT32_MAX : (int)w;
  return DSA_OK;
}

}  // extern "C"
