// Drives the host-only entry points of libdsa.so (row plan, score blocks,
// score width, window size) over random and boundary inputs and checks their
// results; built with the address and undefined-behaviour sanitizers by
// test_host_sanitize.py, so an out-of-bounds access or overflow aborts it.
// Every output buffer is sized exactly, with guard words after it that must
// stay untouched.

#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "dsa.h"

static int failures = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static const int32_t kGuard = 0x5A5A5A5A;

static void plan_rows_trial(std::mt19937& g) {
  const int nreq = std::uniform_int_distribution<int>(0, 40)(g);
  std::vector<int32_t> prior(nreq), fresh(nreq);
  long long total = 0;
  for (int q = 0; q < nreq; ++q) {
    prior[q] = std::uniform_int_distribution<int>(0, 1 << 20)(g);
    fresh[q] = std::uniform_int_distribution<int>(0, 9)(g) == 0
                   ? std::uniform_int_distribution<int>(0, 600)(g)
                   : std::uniform_int_distribution<int>(0, 3)(g);
    total += fresh[q];
  }
  // Exactly sized outputs, then a short buffer that must be refused untouched.
  for (int shortfall = 0; shortfall <= 1; ++shortfall) {
    const int cap = (int)total - shortfall;
    if (cap < 0) continue;
    std::vector<int32_t> req(cap + 4, kGuard), len(cap + 4, kGuard);
    int rows = -1;
    const int st = dsa_plan_rows(nreq, prior.data(), fresh.data(), cap, req.data(), len.data(),
                                 &rows);
    if (shortfall) {
      CHECK(st == DSA_ERR_SHAPE);
      for (int i = 0; i < cap + 4; ++i) CHECK(req[i] == kGuard && len[i] == kGuard);
      continue;
    }
    CHECK(st == DSA_OK && rows == (int)total);
    int r = 0;
    for (int q = 0; q < nreq; ++q)
      for (int i = 0; i < fresh[q]; ++i, ++r) CHECK(req[r] == q && len[r] == prior[q] + i + 1);
    for (int i = cap; i < cap + 4; ++i) CHECK(req[i] == kGuard && len[i] == kGuard);
  }
}

static void plan_blocks_trial(std::mt19937& g) {
  const int rows = std::uniform_int_distribution<int>(0, 500)(g);
  std::vector<int32_t> req(rows);
  int q = 0;
  for (int r = 0; r < rows; ++r) {
    if (std::uniform_int_distribution<int>(0, 5)(g) == 0) ++q;
    req[r] = q;
  }
  const int per = std::uniform_int_distribution<int>(1, 70)(g);
  // Reference count.
  int want = 0;
  for (int r = 0; r < rows;) {
    int e = r + 1;
    while (e < rows && req[e] == req[r] && e - r < per) ++e;
    ++want;
    r = e;
  }
  for (int shortfall = 0; shortfall <= 1; ++shortfall) {
    const int cap = want - shortfall;
    if (cap < 0) continue;
    std::vector<int32_t> blocks(2 * cap + 4, kGuard);
    int nb = -1;
    const int st = dsa_plan_blocks(rows, req.data(), per, cap, blocks.data(), &nb);
    if (shortfall) {
      CHECK(st == DSA_ERR_SHAPE);
      for (size_t i = 0; i < blocks.size(); ++i) CHECK(blocks[i] == kGuard);
      continue;
    }
    CHECK(st == DSA_OK && nb == want);
    int covered = 0;
    for (int b = 0; b < nb; ++b) {
      const int first = blocks[2 * b], n = blocks[2 * b + 1];
      CHECK(first == covered && n >= 1 && n <= per);
      for (int i = 1; i < n; ++i) CHECK(req[first + i] == req[first]);
      covered += n;
    }
    CHECK(covered == rows);
    for (size_t i = 2 * (size_t)cap; i < blocks.size(); ++i) CHECK(blocks[i] == kGuard);
  }
}

static void width_and_windows(std::mt19937& g) {
  const int rows = std::uniform_int_distribution<int>(0, 300)(g);
  std::vector<int32_t> len(rows);
  int mx = 0;
  for (int r = 0; r < rows; ++r) {
    len[r] = std::uniform_int_distribution<int>(0, 1 << 21)(g);
    if (len[r] > mx) mx = len[r];
  }
  int w = -1;
  CHECK(dsa_score_width(rows, len.data(), &w) == DSA_OK);
  CHECK(w >= 64 && w % 64 == 0 && w >= mx && w - mx < 64 + (mx == 0 ? 64 : 0));
  int win = -1;
  const long long bytes = std::uniform_int_distribution<long long>(0, 1LL << 34)(g);
  const int st = dsa_select_window_rows(w, bytes, &win);
  if (bytes < 4LL * w) CHECK(st == DSA_ERR_WORKSPACE);
  else CHECK(st == DSA_OK && (long long)win * w * 4 <= bytes && ((long long)win + 1) * w * 4 > bytes);
}

static void boundaries() {
  int rows = -1, w = -1, nb = -1;
  int32_t p = INT32_MAX, n = 1, req[2], len[2];
  CHECK(dsa_plan_rows(1, &p, &n, 2, req, len, &rows) == DSA_ERR_SHAPE);  // length overflows
  p = INT32_MAX - 1;
  CHECK(dsa_plan_rows(1, &p, &n, 2, req, len, &rows) == DSA_OK && rows == 1 && len[0] == INT32_MAX);
  CHECK(dsa_plan_rows(0, nullptr, nullptr, 0, nullptr, nullptr, &rows) == DSA_OK && rows == 0);
  CHECK(dsa_plan_rows(-1, &p, &n, 2, req, len, &rows) == DSA_ERR_SHAPE);
  CHECK(dsa_plan_rows(1, &p, &n, 2, req, len, nullptr) == DSA_ERR_NULL);
  int32_t big = INT32_MAX - 10;
  CHECK(dsa_score_width(1, &big, &w) == DSA_ERR_SHAPE);
  int32_t neg = -1;
  CHECK(dsa_score_width(1, &neg, &w) == DSA_ERR_SHAPE);
  CHECK(dsa_score_width(0, nullptr, &w) == DSA_OK && w == 64);
  CHECK(dsa_plan_blocks(0, nullptr, 1, 0, nullptr, &nb) == DSA_OK && nb == 0);
  CHECK(dsa_plan_blocks(2, req, 0, 4, len, &nb) == DSA_ERR_SHAPE);
  CHECK(dsa_select_window_rows(1, 1LL << 62, &w) == DSA_OK && w == INT32_MAX);
  for (int s = -7; s <= 1; ++s) CHECK(dsa_status_string(s) != nullptr);
  CHECK(dsa_abi_version() >= 1);
}

int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 2000;
  std::mt19937 g(20260007u);
  boundaries();
  for (int t = 0; t < trials; ++t) {
    plan_rows_trial(g);
    plan_blocks_trial(g);
    width_and_windows(g);
  }
  printf("%d trials, %d failures\n", trials, failures);
  return failures == 0 ? 0 : 1;
}
