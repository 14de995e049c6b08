"""CPU oracle for one paged DSA step (indexer -> top-k -> GQA sparse attention
-> log-sum-exp merge).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP library or its binding and imports
only NumPy.

Every function computes the plain definition of its step in float64, one row
at a time, with no blocking, fusion or reordering beyond what the definition
states. Sources (Megatron-LM pull request 7211, "native dynamic inference for
simplified DSA over GQA"; the commit subjects name the passages):

* rows and their causal lengths -- commit "Treat every query token of a step,
  decode or prefill, as a row ...";
* paged caches read through a block table, 64-key indexer pages -- the PR
  description ("paged KV caches") and commit "--dsa-inference-backend
  flashinfer ..." (indexer cache viewed as 64-key pages, K/V as page-size-1
  slots);
* indexer scores, length-bounded selection, GQA attention per KV group split
  over the top-k slots, and the flash-decoding merge -- commit "Replace the
  CuTe decode kernels with two Triton kernels";
* the selection stays the exact top k -- commit "When a step's context bound
  reaches 64K keys ...";
* valid negative-infinity scores rank ahead of padding -- commit "Replace the
  Triton radix selector with torch.topk ...";
* probabilities stay fp32 through the value reduction -- commit "Restore the
  upstream Blackwell FP32 probability reduction ...".

The indexer's scoring rule is the DeepSeek sparse-attention lightning indexer,
score[s] = sum_h w_h * ReLU(qI_h . kI_s), with one weight per (row, head) and
no further scale. Readings where the pages are silent (each also listed in the
design notes): selected positions are returned in ascending order and padded
with -1; -0.0 ranks equal to +0.0; a decode row's length includes the current
token; query head h reads KV head h // (Hq / Hkv); the attention scale is an
argument (1/sqrt(d) in every workload); the k slots are split into contiguous
slices of ceil(k / S) slots; the log-sum-exp is a natural log.

Every function here is pinned by a CPU test against something other than
itself (brute-force loops, closed forms, hand-worked values, a library
attention routine, invariants); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "row_plan",
    "score_blocks",
    "gather_logical",
    "indexer_scores_row",
    "indexer_scores",
    "topk_row",
    "topk",
    "order_keys",
    "score_histogram_row",
    "split_bounds",
    "attention_split_row",
    "attention_row",
    "merge_row",
    "layer_row",
]


# --------------------------------------------------------------------------
# Row plan
# --------------------------------------------------------------------------


def row_plan(prior, new):
    """Rows of a step, request by request.

    Every new token of a request is a row that attends its causal prefix
    (commit "Treat every query token of a step ... as a row that routes to the
    top-k of its causal prefix"). Token i (0-based) appended after ``prior``
    cached tokens sees positions [0, prior + i], so its length is
    prior + i + 1; a decode request (one new token) gets its full context.
    Returns int32 arrays (row_req, row_len).
    """
    req, length = [], []
    for q, (p, n) in enumerate(zip(prior, new)):
        for i in range(int(n)):
            req.append(q)
            length.append(int(p) + i + 1)
    return np.asarray(req, np.int32), np.asarray(length, np.int32)


def score_blocks(row_req, max_rows):
    """Score blocks: runs of at most ``max_rows`` consecutive rows of one
    request (same commit: "score blocks (consecutive rows of one request)").
    Returns int32 [num_blocks][2] of (first_row, n_rows)."""
    out = []
    r = 0
    n = len(row_req)
    while r < n:
        e = r + 1
        while e < n and row_req[e] == row_req[r] and e - r < max_rows:
            e += 1
        out.append((r, e - r))
        r = e
    return np.asarray(out, np.int32).reshape(-1, 2)


# --------------------------------------------------------------------------
# Paged caches
# --------------------------------------------------------------------------


def gather_logical(cache, block_table_row, length, page):
    """Logical positions [0, length) of one request read through its block
    table: position s lives in physical page block_table_row[s // page] at
    slot s % page. ``cache`` is [num_pages][page][...]."""
    s = np.arange(int(length))
    return cache[np.asarray(block_table_row)[s // page], s % page]


# --------------------------------------------------------------------------
# Indexer
# --------------------------------------------------------------------------


def indexer_scores_row(qI, w, kI):
    """Indexer scores of one row over its logical keys.

    qI [H][D], w [H], kI [L][D] (any float dtype). For every key s:
    score[s] = sum_h w[h] * max(0, qI[h] . kI[s]), computed in float64 and
    returned as float32 (the score buffer's type; a 2048-row by 1M-key buffer
    is sized at 4 bytes a score in commit "Score and select rows in
    windows ..."), with -0.0 written as +0.0.
    """
    q64 = np.asarray(qI, np.float64)
    k64 = np.asarray(kI, np.float64)
    w64 = np.asarray(w, np.float64)
    dots = k64 @ q64.T  # [L][H]
    s = np.maximum(dots, 0.0) @ w64  # [L]
    return (s.astype(np.float32) + np.float32(0.0)).astype(np.float32)


def indexer_scores(qI, w, kI_cache, block_table, row_req, row_len, page):
    """Scores of every row, as a list of float32 arrays of length row_len[r]
    (the indexer reads each row only up to its length)."""
    out = []
    for r in range(len(row_req)):
        q = int(row_req[r])
        kI = gather_logical(kI_cache, block_table[q], int(row_len[r]), page)
        out.append(indexer_scores_row(qI[r], w[r], kI))
    return out


# --------------------------------------------------------------------------
# Length-bounded exact top-k
# --------------------------------------------------------------------------


def topk_row(scores, length, k):
    """Exact top-k of one row over positions [0, length).

    Selects min(k, length) positions with the largest float32 scores, ties to
    the lower position, and returns them in ascending position order followed
    by -1 padding up to k slots. A stable sort of the negated scores puts equal
    scores in ascending position order, so its first k_eff entries are exactly
    that set. -0.0 is ranked as +0.0 (adding +0.0 maps -0.0 to +0.0); a valid
    -inf score is still a selectable position, ahead of every padding slot.
    """
    length = int(length)
    k_eff = min(int(k), length)
    v = np.asarray(scores[:length], np.float32).astype(np.float64) + 0.0
    order = np.argsort(-v, kind="stable")
    sel = np.sort(order[:k_eff])
    out = np.full(int(k), -1, np.int32)
    out[:k_eff] = sel
    return out


def topk(scores_rows, row_len, k):
    """Top-k of every row: int32 [rows][k]."""
    return np.stack([topk_row(s, L, k) for s, L in zip(scores_rows, row_len)]) \
        if len(scores_rows) else np.zeros((0, int(k)), np.int32)


# --------------------------------------------------------------------------
# Score histogram (the selection's exact threshold)
# --------------------------------------------------------------------------


def order_keys(scores):
    """Order-preserving unsigned 32-bit keys of float32 scores, as int64.

    IEEE-754 binary32: a non-negative value's bit pattern grows with the
    value, a negative value's shrinks. Setting the sign bit of non-negative
    patterns and inverting negative ones maps every float32 (-0.0 first made
    +0.0, so the two zeros share a key) to an unsigned integer in the same
    order as the values.
    """
    u = np.asarray(scores, np.float32).view(np.uint32).astype(np.int64)
    u = np.where(u == 0x80000000, 0, u)
    return np.where(u >= 0x80000000, 0xFFFFFFFF - u, u + 0x80000000)


def score_histogram_row(scores, length, bits=12):
    """Counts of a row's first ``length`` scores by the top ``bits`` bits of
    their order keys: int64 [2**bits].

    Commit "When a step's context bound reaches 64K keys, each row now
    thresholds at a sampled score ..." thresholds every row before the exact
    selection; this is the exact counterpart the library uses instead of a
    sample: the bin where the count from the top first reaches k holds the
    k-th largest score (keys of one bin are contiguous in value order).
    """
    length = int(length)
    keys = order_keys(np.asarray(scores, np.float32)[:length])
    return np.bincount(keys >> (32 - int(bits)), minlength=1 << int(bits))


# --------------------------------------------------------------------------
# GQA sparse attention, split over the k slots, and the merge
# --------------------------------------------------------------------------


def split_bounds(k, num_splits):
    """Slot ranges of the splits: contiguous slices of ceil(k / S) slots,
    the last one possibly shorter or empty."""
    c = -(-int(k) // int(num_splits))
    return [(min(int(k), s * c), min(int(k), (s + 1) * c)) for s in range(int(num_splits))]


def attention_split_row(q, k_cache, v_cache, block_table_row, page, idx, scale, num_splits):
    """Per-split attention partials of one row.

    q [Hq][d]; k_cache, v_cache [num_pages][page][Hkv][d], read through the
    request's block table; idx [k] selected logical positions (-1 = padding
    slot, contributes nothing). Query head h reads KV head g = h // (Hq / Hkv);
    the whole group shares the selected keys (commit "Replace the CuTe decode
    kernels ...": one program per KV group reads each selected key and value
    once, and the top-k slots are split across programs). For split sigma over
    its slots:
        z_j = scale * q[h] . K[s_j][g],   m = max z,   l = sum exp(z - m),
        o = sum exp(z_j - m) V[s_j][g] / l,   lse = m + ln l,
    with the probabilities kept at full precision through the value sum
    (commit "Restore the upstream Blackwell FP32 probability reduction").
    An empty split gives o = 0 and lse = -inf.
    Returns part_o [Hq][S][d] and part_lse [Hq][S] in float64.
    """
    q = np.asarray(q, np.float64)
    hq, d = q.shape
    hkv = k_cache.shape[2]
    G = hq // hkv
    idx = np.asarray(idx)
    S = int(num_splits)
    part_o = np.zeros((hq, S, d))
    part_lse = np.full((hq, S), -np.inf)
    bt = np.asarray(block_table_row)
    for sigma, (a, b) in enumerate(split_bounds(len(idx), S)):
        sel = idx[a:b]
        sel = sel[sel >= 0]
        if sel.size == 0:
            continue
        K = np.asarray(k_cache[bt[sel // page], sel % page], np.float64)  # [n][Hkv][d]
        V = np.asarray(v_cache[bt[sel // page], sel % page], np.float64)
        for h in range(hq):
            g = h // G
            z = scale * (K[:, g, :] @ q[h])
            m = z.max()
            p = np.exp(z - m)
            l = p.sum()
            part_o[h, sigma] = (p @ V[:, g, :]) / l
            part_lse[h, sigma] = m + math.log(l)
    return part_o, part_lse


def merge_row(part_o, part_lse):
    """Log-sum-exp merge of split partials (flash decoding, commit "Replace the
    CuTe decode kernels ...": the slices are merged).

    part_o [Hq][S][d], part_lse [Hq][S]. For each head:
        M = max lse,  W = sum exp(lse - M),
        out = sum exp(lse - M) o / W,  out_lse = M + ln W;
    all splits empty gives out = 0, out_lse = -inf.
    """
    part_o = np.asarray(part_o, np.float64)
    part_lse = np.asarray(part_lse, np.float64)
    hq, S, d = part_o.shape
    out = np.zeros((hq, d))
    lse = np.full(hq, -np.inf)
    for h in range(hq):
        M = part_lse[h].max()
        if M == -np.inf:
            continue
        wts = np.exp(part_lse[h] - M)
        W = wts.sum()
        out[h] = (wts @ part_o[h]) / W
        lse[h] = M + math.log(W)
    return out, lse


def attention_row(q, k_cache, v_cache, block_table_row, page, idx, scale):
    """Unsplit attention of one row over its selected keys: (o [Hq][d],
    lse [Hq]). Same definition as ``attention_split_row`` with one split."""
    o, lse = attention_split_row(q, k_cache, v_cache, block_table_row, page, idx, scale, 1)
    return o[:, 0, :], lse[:, 0]


# --------------------------------------------------------------------------
# Whole step for one row
# --------------------------------------------------------------------------


def layer_row(r, row_req, row_len, qI, w, q, kI_cache, k_cache, v_cache, block_table,
              page, k, scale, num_splits=1):
    """Every stage for row r: (scores [L], idx [k], part_o, part_lse, out, lse)."""
    req = int(row_req[r])
    L = int(row_len[r])
    bt = block_table[req]
    s = indexer_scores_row(qI[r], w[r], gather_logical(kI_cache, bt, L, page))
    idx = topk_row(s, L, k)
    po, pl = attention_split_row(q[r], k_cache, v_cache, bt, page, idx, scale, num_splits)
    o, lse = merge_row(po, pl)
    return s, idx, po, pl, o, lse
