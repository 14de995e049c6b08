"""One paged DSA step on the GPU: the row plan, the buffers between the stages,
and the library calls in order on one stream (four, or three with the
attention and merge fused), optionally recorded once into a HIP graph and
replayed.

torch supplies only the device memory and the stream; the row plan comes
from the library's host entry points and every stage runs in its kernels.
The metadata is copied to the device once, at construction, so ``run`` issues
the four launches with no host synchronization.
"""

from __future__ import annotations

import torch

from . import lib


def group_attention_pays(blocks, row_len, topk, block_rows):
    """The step's automatic choice of group attention: there are score blocks
    of 2..8 rows, and none of their rows is longer than 8 x ``topk`` (so a
    block's rows select overlapping keys and their union stays small).
    ``blocks`` is the host block plan ([first row, rows] pairs) or None."""
    if blocks is None or block_rows > 8:
        return False
    multi = [(int(b0), int(n)) for b0, n in blocks if n > 1]
    if not multi:
        return False
    longest = max(int(row_len[b0:b0 + n].max()) for b0, n in multi)
    return longest <= 8 * topk


# Rows longer than this do not fit the one-pass top-k's 32 keys per thread of
# a 1024-thread workgroup; it then holds 64 per thread and its radix passes
# cost twice as much, where the histogram selection only ranks the keys at
# or above the threshold bin.
ONE_PASS_RESIDENT_KEYS = 32768


def histogram_topk_pays(blocks, row_len, one_pass):
    """The step's automatic choice of the histogram top-k (dsa_indexer_scores_hist
    + dsa_topk_hist), for a step without score windows or a forced two-stage
    selection. ``one_pass``: the library would otherwise select in one pass.

    With score blocks of several rows (prefill), the block indexer does not
    count as it scores, so a separate pass counts the written scores; that
    pays only against the two-stage selection of long prefill rows: some
    row of such a block is longer than 2 x ``ONE_PASS_RESIDENT_KEYS`` (the
    one-pass kernel's limit at 64 keys per thread). Measured: 2048 prefill
    rows at 1M context 32.0 -> 31.3 ms; a mixed step whose prefill rows are
    8.5K keys long loses (1642 -> 1714 us).
    Otherwise: the selection runs in one pass and some row is longer than
    ``ONE_PASS_RESIDENT_KEYS``. Measured: ragged batch 64 x 1..65536 193 ->
    179 us; it loses at 32768 keys (+0.7 us), at decode batch 8 (+2 us) and
    against the two-stage selection of 64 rows at 200K (785 vs 788 us)."""
    if len(row_len) == 0:
        return False
    multi = [] if blocks is None else [(int(b0), int(n)) for b0, n in blocks if int(n) > 1]
    if multi:
        longest = max(int(row_len[b0:b0 + n].max()) for b0, n in multi)
        return longest > 2 * ONE_PASS_RESIDENT_KEYS
    return one_pass and int(row_len.max()) > ONE_PASS_RESIDENT_KEYS


class _Seq:
    """Prepared library calls issued one after another on one stream."""

    __slots__ = ("calls",)

    def __init__(self, calls):
        self.calls = calls

    def __call__(self, stream=None):
        for c in self.calls:
            c(stream)


class DsaStep:
    """Buffers and launches for one step of ``inp`` (a StepInputs on a CUDA
    device). ``block_rows`` > 1 groups consecutive rows of a request into
    score blocks for the indexer. ``fused`` runs attention and the merge as
    one launch (dsa_sparse_attn_merged) instead of two; None picks the fused
    launch (with the library's merged split count) unless the batch is small
    enough that the two-launch kernel wants more than 8 splits, and for a
    given ``num_splits`` whenever the merged launch supports it. ``topk_chunk`` > 0 selects in two
    stages over segments of that many positions (dsa_topk_chunked), None
    takes the library's suggestion for the sizes, 0 the one-pass kernel.
    ``score_buffer_bytes`` bounds the score memory: rows are scored and
    selected in windows that fit it (dsa_indexer_topk_windowed), and
    ``scores`` then holds only the last window's rows. ``hist`` has the
    indexer count each row's scores by the top bits of their order keys
    (dsa_indexer_scores_hist) and the top-k start from those counts
    (dsa_topk_hist), which leaves them cleared for the next run; it excludes
    score windows and the two-stage top-k; ``hist=None`` takes it where
    ``histogram_topk_pays`` finds it faster. ``group_attn`` runs the attention
    of the score blocks of several rows (prefill groups, at most 8 rows) over
    the union of their selections on the matrix cores (dsa_group_attn); rows
    from the first of the trailing one-row blocks on (decode rows) keep the
    split attention kernel. ``group_attn=None takes it when the step has such blocks
    and none of their rows is longer than 8 x top-k, where a group's rows
    select overlapping keys (measured: a win at 4.25 x top-k, a loss at
    512 x top-k)."""

    def __init__(self, inp, num_splits: int | None = None, block_rows: int = 1,
                 fused: bool | None = False, topk_chunk: int | None = 0,
                 score_buffer_bytes: int | None = None, hist: bool | None = False,
                 group_attn: bool | None = False):
        wl = inp.wl
        dev = inp.q.device
        self.inp = inp
        self.wl = wl
        req, ln = lib.plan_rows(wl.prior, wl.new)
        self.row_req_host, self.row_len_host = req, ln
        self.rows = len(req)
        self.width = lib.score_width(ln)
        self.total_keys = int(ln.astype("int64").sum())  # the indexer's scheduling hint
        self.row_req = torch.from_numpy(req).to(dev)
        self.row_len = torch.from_numpy(ln).to(dev)
        self.blocks = self.blocks_host = None
        if block_rows > 1:
            self.blocks_host = lib.plan_blocks(req, block_rows)
            self.blocks = torch.from_numpy(self.blocks_host).to(dev)
        shape = (self.rows, wl.hq, wl.hkv, wl.d, wl.topk, inp.q.dtype)
        if fused is None:
            if num_splits:
                fused = num_splits in (1, 2, 4, 6, 8)
            else:
                fused = lib.sparse_attn_splits(*shape) <= 8
        self.fused = fused
        splits_of = lib.sparse_attn_merged_splits if fused else lib.sparse_attn_splits
        self.num_splits = num_splits or splits_of(*shape)
        # Score rows held at once: all of them, or a window that fits the buffer.
        self.window_rows = self.rows
        if score_buffer_bytes is not None:
            self.window_rows = min(self.rows, lib.select_window_rows(self.width, score_buffer_bytes))
        if hist and (score_buffer_bytes is not None or topk_chunk):
            raise ValueError("the histogram top-k does not combine with score windows or two stages")
        suggested = topk_chunk
        if suggested is None:
            # The suggestion for a window's rows, at the batch's fill.
            window_keys = self.total_keys * self.window_rows // max(1, self.rows)
            suggested = lib.topk_chunk_suggest(self.window_rows, self.width, wl.topk, window_keys)
        if hist is None:
            # Not with score windows or a two-stage selection the caller asked for.
            hist = (score_buffer_bytes is None and not topk_chunk
                    and histogram_topk_pays(self.blocks_host, ln, not suggested))
        topk_chunk = 0 if hist else suggested
        self.use_hist = hist
        self.topk_chunk = topk_chunk
        self.windowed = score_buffer_bytes is not None
        self.scores = torch.empty(self.window_rows, self.width, dtype=torch.float32, device=dev)
        self.idx = torch.empty(self.rows, wl.topk, dtype=torch.int32, device=dev)
        self.cand = None
        if topk_chunk:
            self.cand = torch.empty(lib.topk_chunked_slots(self.window_rows, self.width, wl.topk,
                                                           topk_chunk), dtype=torch.int32, device=dev)
        parts = 0 if fused else self.rows
        self.part_o = torch.empty(parts, wl.hq, self.num_splits, wl.d, dtype=torch.float32,
                                  device=dev)
        self.part_lse = torch.empty(parts, wl.hq, self.num_splits, dtype=torch.float32,
                                    device=dev)
        self.out = torch.empty(self.rows, wl.hq, wl.d, dtype=inp.q.dtype, device=dev)
        self.out_lse = torch.empty(self.rows, wl.hq, dtype=torch.float32, device=dev)
        # Group attention: the blocks before the trailing one-row blocks.
        self.group_rows = 0
        self.groups = None
        if group_attn is None:
            group_attn = group_attention_pays(self.blocks_host, ln, wl.topk, block_rows)
        if group_attn:
            if self.blocks_host is None or block_rows > 8:
                raise ValueError("group attention needs score blocks of at most 8 rows")
            nb = len(self.blocks_host)
            tail = nb
            while tail > 0 and self.blocks_host[tail - 1][1] == 1:
                tail -= 1
            self.group_rows = int(self.blocks_host[tail][0]) if tail < nb else self.rows
            if tail > 0:
                self.groups = torch.from_numpy(self.blocks_host[:tail].copy()).to(dev)
        # Zero once; the top-k clears the counts it read.
        self.hist = (torch.zeros(self.rows, lib.HIST_BINS, dtype=torch.int32, device=dev)
                     if hist else None)

        self._prepare()

    def _prepare(self):
        """Checks and marshals every library call of the step once; each stage
        then only launches (the binding's per-call tensor checks would
        otherwise cost more host time than a small step takes on the GPU)."""
        i, wl = self.inp, self.wl
        self._calls = {"indexer": None, "topk": None, "attention": None, "merge": None}
        if self.windowed:
            # Indexer and top-k as one call that alternates them window by window.
            self._calls["indexer"] = lib.indexer_topk_windowed(
                i.qI, i.w, i.kI_cache, i.block_table, self.row_req, self.row_len, self.width,
                wl.page, wl.topk, self.scores, self.idx, topk_chunk=self.topk_chunk,
                cand=self.cand, prepare=True, blocks=self.blocks, blocks_host=self.blocks_host)
        elif self.use_hist:
            self._calls["indexer"] = lib.indexer_scores_hist(
                i.qI, i.w, i.kI_cache, i.block_table, self.row_req, self.row_len, self.scores,
                self.hist, wl.page, blocks=self.blocks, total_keys=self.total_keys, prepare=True)
            self._calls["topk"] = lib.topk_hist(self.scores, self.row_len, self.hist, wl.topk,
                                                self.idx, total_keys=self.total_keys, prepare=True)
        else:
            self._calls["indexer"] = lib.indexer_scores(
                i.qI, i.w, i.kI_cache, i.block_table, self.row_req, self.row_len, self.scores,
                wl.page, blocks=self.blocks, total_keys=self.total_keys, prepare=True)
            if self.topk_chunk:
                self._calls["topk"] = lib.topk_chunked(self.scores, self.row_len, wl.topk,
                                                       self.topk_chunk, self.cand, self.idx,
                                                       prepare=True)
            else:
                self._calls["topk"] = lib.topk(self.scores, self.row_len, wl.topk, self.idx,
                                               total_keys=self.total_keys, prepare=True)
        if self.groups is not None:
            calls = [lib.group_attn(i.q, i.k_cache, i.v_cache, i.block_table, self.row_req,
                                    self.idx, self.groups, wl.page, wl.attn_scale, self.out,
                                    self.out_lse, prepare=True)]
            g0 = self.group_rows
            if g0 < self.rows:
                # The decode rows after the groups, on the split attention kernel.
                sl = slice(g0, self.rows)
                splits = lib.sparse_attn_merged_splits(self.rows - g0, wl.hq, wl.hkv, wl.d,
                                                       wl.topk, i.q.dtype)
                calls.append(lib.sparse_attn_merged(
                    i.q[sl], i.k_cache, i.v_cache, i.block_table, self.row_req[sl], self.idx[sl],
                    wl.page, wl.attn_scale, splits, self.out[sl], self.out_lse[sl], prepare=True))
            self._calls["attention"] = _Seq(calls)
        elif self.fused:
            self._calls["attention"] = lib.sparse_attn_merged(
                i.q, i.k_cache, i.v_cache, i.block_table, self.row_req, self.idx, wl.page,
                wl.attn_scale, self.num_splits, self.out, self.out_lse, prepare=True)
        else:
            self._calls["attention"] = lib.sparse_attn(
                i.q, i.k_cache, i.v_cache, i.block_table, self.row_req, self.idx, wl.page,
                wl.attn_scale, self.num_splits, self.part_o, self.part_lse, prepare=True)
            self._calls["merge"] = lib.merge(self.part_o, self.part_lse, self.out, self.out_lse,
                                             prepare=True)
        self._seq = [c for c in self._calls.values() if c is not None]

    # The four stages, each one library call (with score windows, indexer and
    # top-k are one call; with the fused attention, attention and merge).
    def _stage(self, name, stream):
        c = self._calls[name]
        if c is not None:
            c(stream)

    def indexer(self, stream=None):
        self._stage("indexer", stream)

    def topk(self, stream=None):
        self._stage("topk", stream)

    def attention(self, stream=None):
        self._stage("attention", stream)

    def merge(self, stream=None):
        self._stage("merge", stream)

    def run(self, stream=None):
        h = lib._stream(stream)  # resolved once for the step's launches
        for c in self._seq:
            c(h)
        return self.out

    def capture(self):
        """Records the step's launches into a HIP graph (torch's graph capture
        on ROCm) and returns it; ``graph.replay()`` runs them again on the same
        buffers. The kernels read the metadata (lengths, request ids, block
        tables, selected positions) from device memory when they run, so those
        may change between replays as long as the score width and row count
        stay the same. Nothing the step records clears memory with a memset
        node: every output is written by a kernel."""
        import torch

        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()  # one eager pass on the capturing side before recording
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            self.run()
        return graph
