"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Scores and indices must match bit for bit; attention partials and outputs
within max-abs 2e-2 (bf16 inputs) or 1e-5 (fp32 inputs), the log-sum-exp
within 1e-3 / 1e-5. Small workloads are checked on every row; the large ones
(headline, ragged, mixed, 64 x 200K decode, 2048-row prefill at 1M context)
run at full size in the launch configuration the benchmark times: every row
of the headline and ragged batches, every decode row and every 64th prefill
row of the mixed step against the oracle (sampled rows of the two largest),
and every row checked for the properties of a correct selection. Alternative paths of the library (score
blocks and the block indexer, two-stage top-k, row windows, the fused merge,
graph replay, the scheduling hints) are checked bit for bit against the
default ones.
"""

import sys

import numpy as np
import pytest
import torch

from dsa_check import CANARY, check_properties, check_row, oracle_row, run_step
from oracle import dsa_oracle as O
from sparse_attention_decode_02_amd import inputs as I
from sparse_attention_decode_02_amd.step import DsaStep

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_attention_decode_02_amd.lib  # noqa: F401  (raises if the library is missing)
    yield
    torch.cuda.empty_cache()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _host_inputs(wl):
    return I.to_device(I.generate(wl, "cpu"), "cuda")


def _check_all(step):
    errs = [check_row(step, r) for r in range(step.rows)]
    check_properties(step)
    return {k: max(e[k] for e in errs) for k in errs[0]}


# --------------------------------------------------------------------------
# Small workloads, every row
# --------------------------------------------------------------------------


@pytest.mark.parametrize("S", [1, 2, 3, 16])
def test_tiny_every_row(S):
    _say(f"tiny fp32, splits {S}")
    step = run_step(_host_inputs(I.tiny()), num_splits=S)
    e = _check_all(step)
    _say(f"  max errors {e}")


def test_decode_b8_every_row():
    _say("decode batch 8 x 4096, bf16")
    step = run_step(_host_inputs(I.decode()))
    e = _check_all(step)
    _say(f"  splits {step.num_splits}, max errors {e}")


def _small_mixed(seed=7, topk=256):
    prior = (700, 300, 0, 62, 63, 64, 254, 255, 256, 2999, 5000)
    new = (37, 5, 1, 1, 1, 1, 1, 1, 1, 1, 1)
    return I.custom(I.decode(), name="small_mixed", hq=16, hkv=2, topk=topk, prior=prior,
                    new=new, seed=seed)


@pytest.mark.parametrize("block_rows", [1, 8])
@pytest.mark.parametrize("S", [1, 4])
def test_small_mixed_every_row(block_rows, S):
    _say(f"small mixed bf16, block_rows {block_rows}, splits {S}")
    step = run_step(_host_inputs(_small_mixed()), num_splits=S, block_rows=block_rows)
    lens = step.row_len_host.tolist()
    assert {1, 63, 64, 65, 255, 256, 257} <= set(lens)  # around k and the page size
    e = _check_all(step)
    _say(f"  max errors {e}")


@pytest.mark.parametrize("S", [1, 2, 5, 8, 256])
def test_split_counts(S):
    _say(f"splits {S}")
    wl = _small_mixed(seed=11)
    step = run_step(_host_inputs(wl), num_splits=S)
    for r in (0, 36, 40, step.rows - 1):
        check_row(step, r)


@pytest.mark.parametrize("S,fused", [(1, False), (3, False), (1, True), (2, True)])
def test_attention_splits_over_several_spans(S, fused):
    """Splits of more than 512 slots: the attention kernels resolve a split's
    positions to cache rows 256 or 512 at a time (the matrix-core kernel, by
    workgroup size) or 512 at a time (the vector kernel), so these walk
    several spans, the last one partial, with short rows' padding in the
    later spans."""
    _say(f"attention over several spans, splits {S}, fused {fused}")
    step = run_step(_host_inputs(_small_mixed(seed=61, topk=1024)), num_splits=S, fused=fused)
    e = _check_all(step)
    _say(f"  max errors {e}")


@pytest.mark.parametrize("S", [1, 2, 4, 6, 8])
def test_merged_matches_split_then_merge_bitwise(S):
    """dsa_sparse_attn_merged writes exactly what dsa_sparse_attn + dsa_merge
    write, and both match the oracle."""
    _say(f"merged attention, splits {S}")
    inp = _host_inputs(_small_mixed(seed=13))
    two = run_step(inp, num_splits=S)
    one = run_step(inp, num_splits=S, fused=True)
    assert torch.equal(one.idx, two.idx)
    assert torch.equal(one.out.view(torch.int16), two.out.view(torch.int16))
    assert torch.equal(one.out_lse.view(torch.int32), two.out_lse.view(torch.int32))
    for r in (0, 36, 40, one.rows - 1):
        check_row(one, r)


@pytest.mark.parametrize("v", [("f32", 16, 4, 1, 64, 4, 32, 16), ("bf16", 32, 32, 2, 128, 64, 128, 64),
                               ("bf16", 16, 16, 4, 64, 32, 64, 128)], ids=lambda v: "-".join(map(str, v)))
def test_merged_shapes(v):
    dt, page, hq, hkv, d, hi, di, topk = v
    wl = I.custom(I.tiny(), name="variant", dtype=dt, page=page, hq=hq, hkv=hkv, d=d, hi=hi,
                  di=di, topk=topk, prior=(3, 150, 700, 40), new=(1, 1, 1, 6), seed=77)
    inp = _host_inputs(wl)
    for S in (1, 2, 4, 6):
        two = run_step(inp, num_splits=S)
        one = run_step(inp, num_splits=S, fused=True)
        dtv = torch.int16 if dt == "bf16" else torch.int32
        assert torch.equal(one.out.view(dtv), two.out.view(dtv)), S
        _check_all(one)


VARIANTS = [
    # dtype, page, hq, hkv, d, hi, di, topk
    ("bf16", 64, 8, 8, 128, 32, 128, 64),
    ("bf16", 32, 16, 4, 64, 64, 64, 64),
    ("bf16", 16, 32, 16, 64, 32, 64, 128),
    ("bf16", 64, 16, 1, 128, 64, 128, 100),
    ("bf16", 128, 32, 2, 128, 64, 128, 64),
    # the matrix-core attention's shape (8 query heads per KV group, d 128)
    # at other page sizes, KV group counts and top-k not a multiple of 16
    ("bf16", 16, 8, 1, 128, 64, 128, 100),
    ("bf16", 128, 64, 8, 128, 64, 128, 48),
    ("bf16", 32, 16, 2, 128, 32, 64, 257),
    ("f32", 16, 4, 1, 64, 4, 32, 16),
    ("f32", 8, 8, 4, 128, 64, 128, 40),
    ("f32", 64, 16, 2, 64, 17, 64, 64),
    ("f32", 32, 16, 1, 128, 1, 32, 33),
]


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: "-".join(map(str, v)))
def test_supported_shapes(v):
    dt, page, hq, hkv, d, hi, di, topk = v
    _say(f"shape variant {v}")
    wl = I.custom(I.tiny(), name="variant", dtype=dt, page=page, hq=hq, hkv=hkv, d=d, hi=hi,
                  di=di, topk=topk, prior=(3, 150, 700, 40), new=(1, 1, 1, 6), seed=1000 + VARIANTS.index(v))
    step = run_step(_host_inputs(wl))
    _check_all(step)


# --------------------------------------------------------------------------
# Edge cases fed straight to the stages
# --------------------------------------------------------------------------


def _topk_case_rows(width, k):
    rng = np.random.default_rng(5)
    rows = []
    rows.append(("all equal", np.full(5000, 7.5, np.float32)))
    rows.append(("increasing", np.arange(4000, dtype=np.float32)))
    rows.append(("decreasing", np.arange(4000, 0, -1).astype(np.float32)))
    sc = rng.integers(-3, 4, 6000).astype(np.float32)
    sc[rng.integers(0, 6000, 500)] = np.inf
    sc[rng.integers(0, 6000, 500)] = -np.inf
    rows.append(("infinities", sc))
    sc = np.where(rng.random(5000) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    sc[rng.integers(0, 5000, 100)] = 1.0
    rows.append(("signed zeros", sc))
    rows.append(("all -inf", np.full(3000, -np.inf, np.float32)))
    rows.append(("empty", np.zeros(0, np.float32)))
    rows.append(("one", np.asarray([3.0], np.float32)))
    rows.append(("k-1", rng.standard_normal(k - 1).astype(np.float32)))
    rows.append(("k", rng.standard_normal(k).astype(np.float32)))
    rows.append(("k+1", rng.standard_normal(k + 1).astype(np.float32)))
    rows.append(("two values", np.where(rng.random(9000) < 0.3, 1.0, 2.0).astype(np.float32)))
    rows.append(("normal", rng.standard_normal(30000).astype(np.float32)))
    rows.append(("chunked ties", (rng.integers(0, 2000, 40000) / 2).astype(np.float32)))
    rows.append(("chunked long", (rng.integers(0, 50000, width) / 4).astype(np.float32)))
    rows.append(("chunked huge range", (rng.standard_normal(70000) * 1e30).astype(np.float32)))
    rows.append(("denormals", (rng.integers(1, 100, 8000) * np.float32(1e-45)).astype(np.float32)))
    rows.append(("mixed signs", rng.standard_normal(32768).astype(np.float32) * 1e-3))
    # indexer-like scores: multiples of 0.5 around 2240, a few dozen keys tied
    # with the threshold digit (resolved by direct ranking)
    rows.append(("indexer-like", np.maximum(0, np.round(rng.normal(2240, 400, 32768) * 2) / 2)
                 .astype(np.float32)))
    # rows at the ranking limits: every key a candidate, with repeated values
    rows.append(("short ranked", (rng.integers(0, 40, 511) / 4).astype(np.float32)))
    rows.append(("short ranked mixed signs", rng.standard_normal(300).astype(np.float32)))
    # a whole 65536-key chunk tied with the threshold (the emit's counts must
    # not share one word): all equal, all zero (rectified scores), and 65536
    # zeros ahead of a few positive scores
    rows.append(("70000 equal", np.full(70000, 7.5, np.float32)))
    rows.append(("70000 zeros", np.zeros(70000, np.float32)))
    rows.append(("65536 zeros then positives",
                 np.concatenate([np.zeros(65536, np.float32),
                                 (rng.random(100) + 1).astype(np.float32)])))
    return rows


@pytest.mark.parametrize("k", [1, 16, 2048])
@pytest.mark.parametrize("copies,width", [(1, 70016), (13, 70016), (1, 4096), (1, 8192), (3, 16384)],
                         ids=["few-rows", "many-rows", "w4096", "w8192", "w16384"])
def test_topk_edges(k, copies, width):
    """Edge rows against the oracle. A batch of few wide rows runs the
    64-keys-per-thread kernel, a batch of more rows than CUs the 32-keys one;
    score widths up to 16384 run the 512-thread kernels (rows cut to the
    width)."""
    from sparse_attention_decode_02_amd import lib
    if k > width:
        pytest.skip("k > width")
    cases = [(n, sc[:width]) for n, sc in _topk_case_rows(width, k)] * copies
    _say(f"top-k edges, k {k}, {len(cases)} rows")
    scores = np.full((len(cases), width), np.nan, np.float32)
    lens = np.zeros(len(cases), np.int32)
    for i, (_, sc) in enumerate(cases):
        scores[i, : len(sc)] = sc
        lens[i] = len(sc)
    s_d = torch.from_numpy(scores).cuda()
    l_d = torch.from_numpy(lens).cuda()
    idx = torch.full((len(cases), k), -7, dtype=torch.int32, device="cuda")
    lib.topk(s_d, l_d, k, idx)
    got = idx.cpu().numpy()
    for i, (name, sc) in enumerate(cases):
        want = O.topk_row(sc, len(sc), k)
        assert np.array_equal(got[i], want), f"{name}: first diff at {np.flatnonzero(got[i] != want)[:5]}"


def _oracle_hist(sc, L):
    return O.score_histogram_row(sc, L).astype(np.int64)


@pytest.mark.parametrize("width", [70016, 16384, 4096])
def test_score_hist_matches_oracle(width):
    """dsa_score_hist counts every edge row's scores exactly as the oracle."""
    from sparse_attention_decode_02_amd import lib
    cases = [(n, sc[:width]) for n, sc in _topk_case_rows(width, 2048)]
    scores = np.full((len(cases), width), np.nan, np.float32)
    lens = np.zeros(len(cases), np.int32)
    for i, (_, sc) in enumerate(cases):
        scores[i, : len(sc)] = sc
        lens[i] = len(sc)
    hist = torch.full((len(cases), lib.HIST_BINS), 7, dtype=torch.int32, device="cuda")
    lib.score_hist(torch.from_numpy(scores).cuda(), torch.from_numpy(lens).cuda(), hist)
    got = hist.cpu().numpy().astype(np.int64)
    for i, (name, sc) in enumerate(cases):
        assert np.array_equal(got[i], _oracle_hist(sc, len(sc))), name


def test_score_hist_counter_bound():
    """dsa_score_hist at the largest count one of its 16-bit LDS counters can
    take: 1024 rows of 62 x 8192 positions give two workgroups a row, each
    counting 31 chunks, and rows of equal scores put all of a copy's keys in
    one bin (64 threads x 32 keys x 31 = 63488); random rows beside them
    match the oracle's histogram."""
    from sparse_attention_decode_02_amd import lib
    rows, width = 1024, 62 * 8192
    scores = torch.ones(rows, width, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(47)
    rand = [rng.standard_normal(width).astype(np.float32) for _ in range(4)]
    for i, sc in enumerate(rand):
        scores[rows - 1 - i] = torch.from_numpy(sc).cuda()
    lens = torch.full((rows,), width, dtype=torch.int32, device="cuda")
    hist = torch.full((rows, lib.HIST_BINS), 7, dtype=torch.int32, device="cuda")
    lib.score_hist(scores, lens, hist)
    got = hist.cpu().numpy().astype(np.int64)
    del scores
    want = _oracle_hist(np.ones(1, np.float32), 1) * width
    for r in range(rows - 4):
        assert np.array_equal(got[r], want), r
    for i, sc in enumerate(rand):
        assert np.array_equal(got[rows - 1 - i], _oracle_hist(sc, width)), i


@pytest.mark.parametrize("k", [1, 16, 2048])
@pytest.mark.parametrize("copies,width", [(1, 70016), (13, 70016), (1, 4096), (1, 8192), (3, 16384)],
                         ids=["few-rows", "many-rows", "w4096", "w8192", "w16384"])
def test_topk_hist_edges(k, copies, width):
    """The histogram-driven selection on every edge row against the oracle;
    the histogram comes back cleared. Rows whose candidates overflow the
    on-chip list (long fully tied rows) take the narrowing passes and the
    emit over the row."""
    from sparse_attention_decode_02_amd import lib
    if k > width:
        pytest.skip("k > width")
    cases = [(n, sc[:width]) for n, sc in _topk_case_rows(width, k)] * copies
    _say(f"histogram top-k edges, k {k}, {len(cases)} rows")
    scores = np.full((len(cases), width), np.nan, np.float32)
    lens = np.zeros(len(cases), np.int32)
    for i, (_, sc) in enumerate(cases):
        scores[i, : len(sc)] = sc
        lens[i] = len(sc)
    s_d = torch.from_numpy(scores).cuda()
    l_d = torch.from_numpy(lens).cuda()
    hist = torch.zeros((len(cases), lib.HIST_BINS), dtype=torch.int32, device="cuda")
    lib.score_hist(s_d, l_d, hist)
    idx = torch.full((len(cases), k), -7, dtype=torch.int32, device="cuda")
    lib.topk_hist(s_d, l_d, hist, k, idx, total_keys=int(lens.astype(np.int64).sum()))
    torch.cuda.synchronize()
    assert not bool(hist.any()), "the histogram was not cleared"
    got = idx.cpu().numpy()
    for i, (name, sc) in enumerate(cases):
        want = O.topk_row(sc, len(sc), k)
        assert np.array_equal(got[i], want), f"{name}: first diff at {np.flatnonzero(got[i] != want)[:5]}"


def test_topk_hist_without_a_matching_histogram():
    """A histogram that does not count the row (here all zero) makes the
    selection rank the row from scratch: still the oracle's indices."""
    from sparse_attention_decode_02_amd import lib
    cases, s_d, l_d = _edge_batch(2048)
    hist = torch.zeros((len(cases), lib.HIST_BINS), dtype=torch.int32, device="cuda")
    idx = torch.full((len(cases), 2048), -7, dtype=torch.int32, device="cuda")
    lib.topk_hist(s_d, l_d, hist, 2048, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for i, (name, sc) in enumerate(cases):
        assert np.array_equal(got[i], O.topk_row(sc, len(sc), 2048)), name


@pytest.mark.parametrize("wl_fn,block_rows", [(I.decode, 1), (lambda: _small_mixed(seed=43), 8),
                                              (lambda: _small_mixed(seed=44), 1), (I.tiny, 1)],
                         ids=["decode", "blocks", "small-mixed", "tiny-f32"])
def test_indexer_hist_and_step(wl_fn, block_rows):
    """dsa_indexer_scores_hist leaves the oracle's histogram of every row
    (fused in the row kernel, counted after the block kernel or the fp32
    kernel), and the histogram step gives the default step's bits."""
    inp = _host_inputs(wl_fn())
    ref = run_step(inp, block_rows=block_rows, fused=None)
    step = DsaStep(inp, block_rows=block_rows, fused=None, hist=True)
    step.scores.view(torch.int32).fill_(CANARY)
    step.indexer()
    torch.cuda.synchronize()
    h = step.hist.cpu().numpy().astype(np.int64)
    for r in range(step.rows):
        L = int(step.row_len_host[r])
        sc = step.scores[r, :L].cpu().numpy()
        assert np.array_equal(h[r], _oracle_hist(sc, L)), r
    step.topk()
    step.attention()
    step.merge()
    torch.cuda.synchronize()
    assert not bool(step.hist.any())
    for x, y in ((ref.idx, step.idx), (ref.out, step.out), (ref.out_lse, step.out_lse)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    for r in range(0, step.rows, max(1, step.rows // 6)):
        check_row(step, r)
    step.run()  # a second step on the cleared counts
    torch.cuda.synchronize()
    assert torch.equal(ref.idx, step.idx) and not bool(step.hist.any())


@pytest.mark.parametrize("k", [16, 2048])
def test_topk_hint_many_short_rows(k):
    """A batch of at least four rows per CU, short on average: with the
    row-length hint the selection runs in the small-workgroup kernel whatever
    the width; the edge rows (up to 70016 long) and sampled short rows
    against the oracle, every row bit for bit against the unhinted call."""
    from sparse_attention_decode_02_amd import lib
    width = 70016
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    edge = _topk_case_rows(width, k)
    n = max(4 * cus, 1024) + len(edge)
    rng = np.random.default_rng(11)
    lens = rng.integers(1, 9000, n).astype(np.int32)
    scores = np.full((n, width), np.nan, np.float32)
    short = rng.integers(-64, 64, (n, 9000)).astype(np.float32)  # small integers: many ties
    for i in range(n):
        scores[i, : lens[i]] = short[i, : lens[i]]
    for i, (_, sc) in enumerate(edge):
        scores[i, : len(sc)] = sc
        scores[i, len(sc):] = np.nan
        lens[i] = len(sc)
    total = int(lens.astype(np.int64).sum())
    assert n >= 4 * cus and total <= 16384 * n
    _say(f"top-k with the hint, k {k}, {n} rows, mean length {total / n:.0f}")
    s_d = torch.from_numpy(scores).cuda()
    l_d = torch.from_numpy(lens).cuda()
    plain = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
    hinted = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
    lib.topk(s_d, l_d, k, plain)
    lib.topk(s_d, l_d, k, hinted, total_keys=total)
    torch.cuda.synchronize()
    assert torch.equal(hinted, plain)
    got = hinted.cpu().numpy()
    for i in list(range(len(edge))) + [len(edge), n // 2, n - 1]:
        sc = scores[i, : lens[i]]
        want = O.topk_row(sc, int(lens[i]), k)
        assert np.array_equal(got[i], want), f"row {i}: first diff at {np.flatnonzero(got[i] != want)[:5]}"


def _edge_batch(k):
    width = 70016
    cases = _topk_case_rows(width, k)
    scores = np.full((len(cases), width), np.nan, np.float32)
    lens = np.zeros(len(cases), np.int32)
    for i, (_, sc) in enumerate(cases):
        scores[i, : len(sc)] = sc
        lens[i] = len(sc)
    return cases, torch.from_numpy(scores).cuda(), torch.from_numpy(lens).cuda()


@pytest.mark.parametrize("k,chunk", [(1, 4), (16, 16), (16, 100), (16, 4096), (2048, 2048),
                                     (2048, 8192), (2048, 40000), (16, 70000), (2048, 70000)])
def test_topk_chunked_edges(k, chunk):
    """The two-stage selection (segment winners, then the row's top-k among
    them) against the oracle, and bit for bit against the one-pass kernel."""
    from sparse_attention_decode_02_amd import lib
    cases, s_d, l_d = _edge_batch(k)
    _say(f"chunked top-k edges, k {k}, chunk {chunk}, {len(cases)} rows")
    rows, width = s_d.shape
    one = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    lib.topk(s_d, l_d, k, one)
    cand = torch.full((lib.topk_chunked_slots(rows, width, k, chunk),), -9, dtype=torch.int32,
                      device="cuda")
    two = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    lib.topk_chunked(s_d, l_d, k, chunk, cand, two)
    got = two.cpu().numpy()
    for i, (name, sc) in enumerate(cases):
        want = O.topk_row(sc, len(sc), k)
        assert np.array_equal(got[i], want), f"{name}: first diff at {np.flatnonzero(got[i] != want)[:5]}"
    assert torch.equal(two, one)


@pytest.mark.parametrize("window_rows,topk_chunk", [(1, 0), (5, 0), (64, 0), (5, 256), (7, 1024)])
def test_windowed_matches_full_batch(window_rows, topk_chunk):
    """Scores and selection in row windows through a bounded buffer give the
    indices of the whole-batch calls, which the oracle checks row by row."""
    from sparse_attention_decode_02_amd import lib
    wl = _small_mixed(seed=21)
    step = run_step(_host_inputs(wl), num_splits=4)
    _say(f"windowed indexer + top-k, {window_rows} rows per window, chunk {topk_chunk}")
    inp = step.inp
    buf = torch.empty(window_rows * step.width, dtype=torch.float32, device="cuda")
    assert lib.select_window_rows(step.width, buf.numel() * 4) == window_rows
    cand = None
    if topk_chunk:
        n = lib.topk_chunked_slots(min(window_rows, step.rows), step.width, wl.topk, topk_chunk)
        cand = torch.empty(n, dtype=torch.int32, device="cuda")
    idx = torch.full_like(step.idx, -7)
    lib.indexer_topk_windowed(inp.qI, inp.w, inp.kI_cache, inp.block_table, step.row_req,
                              step.row_len, step.width, wl.page, wl.topk, buf, idx,
                              topk_chunk=topk_chunk, cand=cand)
    torch.cuda.synchronize()
    assert torch.equal(idx, step.idx)
    for r in (0, 36, 37, step.rows - 1):
        check_row(step, r)


@pytest.mark.parametrize("kw", [dict(topk_chunk=1024), dict(score_buffer_bytes=6 * 5120 * 4),
                                dict(score_buffer_bytes=6 * 5120 * 4, topk_chunk=512),
                                dict(topk_chunk=None),
                                dict(score_buffer_bytes=16 * 5120 * 4, block_rows=8),
                                dict(score_buffer_bytes=9 * 5120 * 4, block_rows=4, topk_chunk=512)],
                         ids=["chunked", "windowed", "windowed-chunked", "suggested",
                              "windowed-blocks", "windowed-blocks-chunked"])
def test_step_variants_bit_identical(kw):
    """The step with the two-stage top-k and/or score windows gives the
    default step's indices and outputs bit for bit."""
    inp = _host_inputs(_small_mixed(seed=23, topk=512))
    ref = run_step(inp, num_splits=4)
    outs = [t.clone() for t in (ref.idx, ref.out, ref.out_lse)]
    step = DsaStep(inp, num_splits=4, **kw)
    _say(f"step variant {kw}: window rows {step.window_rows}, top-k chunk {step.topk_chunk}")
    step.run()
    torch.cuda.synchronize()
    for a, b in zip(outs, (step.idx, step.out, step.out_lse)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_step_automatic_histogram_topk():
    """With a row longer than the one-pass top-k holds at 32 keys per thread
    and no prefill blocks, the step's automatic choice takes the histogram
    selection, and it gives the one-pass step's indices and outputs bit for
    bit (and the oracle's on the long row); with prefill blocks only when
    their rows are longer than the one-pass top-k holds at all (then the
    two-stage step's bits)."""
    wl = I.custom(I.decode(), name="long_row", hq=16, hkv=2, topk=256,
                  prior=(40000, 300, 5000), new=(1, 1, 1), seed=29)
    inp = _host_inputs(wl)
    ref = run_step(inp, num_splits=4)
    outs = [t.clone() for t in (ref.idx, ref.out, ref.out_lse)]
    step = run_step(inp, num_splits=4, hist=None, topk_chunk=None)
    _say(f"automatic top-k: histogram {step.use_hist}, chunk {step.topk_chunk}")
    assert step.use_hist and not step.topk_chunk
    for a, b in zip(outs, (step.idx, step.out, step.out_lse)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    check_row(step, 0)
    # with a prefill block the automatic choice keeps the one-pass selection
    blk = DsaStep(_host_inputs(_small_mixed(seed=29)), block_rows=8, hist=None, topk_chunk=None)
    assert not blk.use_hist
    # ... unless a block's rows are longer than the one-pass kernel holds:
    # then the histogram selection replaces the two-stage one, same bits
    wl2 = I.custom(I.decode(), name="long_block", hq=16, hkv=2, topk=256,
                   prior=(65600, 300), new=(3, 1), seed=31)
    inp2 = _host_inputs(wl2)
    two = run_step(inp2, num_splits=4, block_rows=8, topk_chunk=32768)
    outs2 = [t.clone() for t in (two.idx, two.out, two.out_lse)]
    auto = run_step(inp2, num_splits=4, block_rows=8, hist=None, topk_chunk=None)
    _say(f"automatic top-k, long prefill block: histogram {auto.use_hist}, chunk {auto.topk_chunk}")
    assert auto.use_hist and not auto.topk_chunk
    for a, b in zip(outs2, (auto.idx, auto.out, auto.out_lse)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    check_row(auto, 1)


def test_windowed_fp32_tiny():
    from sparse_attention_decode_02_amd import lib
    wl = I.tiny()
    step = run_step(_host_inputs(wl))
    inp = step.inp
    buf = torch.empty(step.width, dtype=torch.float32, device="cuda")  # one row per window
    idx = torch.full_like(step.idx, -7)
    lib.indexer_topk_windowed(inp.qI, inp.w, inp.kI_cache, inp.block_table, step.row_req,
                              step.row_len, step.width, wl.page, wl.topk, buf, idx)
    torch.cuda.synchronize()
    assert torch.equal(idx, step.idx)
    for r in range(step.rows):
        check_row(step, r)


def _gapped_idx(step, rng):
    """Caller-given selections with -1 anywhere (allowed by the contract):
    a leading run of more than one 32-slot tile, a fully empty quarter, gaps
    in the middle; valid slots hold distinct positions below the row length."""
    k = step.wl.topk
    out = np.full((step.rows, k), -1, np.int32)
    for r in range(step.rows):
        L = int(step.row_len_host[r])
        n = min(L, k)
        pos = rng.permutation(L)[:n].astype(np.int32)
        slots = np.arange(k)
        keep = (slots >= 40) & ~((slots >= k // 4) & (slots < k // 2))
        keep &= ~((slots >= 3 * k // 4 + 7) & (slots < 3 * k // 4 + 45))
        keep_slots = slots[keep][:n]
        out[r, keep_slots] = pos[: len(keep_slots)]
    return out


def _oracle_attention(step, r, idx_row, S):
    inp, wl = step.inp, step.wl
    req = int(step.row_req_host[r])
    bt = inp.block_table[req]
    valid = idx_row >= 0
    n = int(valid.sum())
    kc = np.zeros((max(n, 1), 1, wl.hkv, wl.d))
    vc = np.zeros((max(n, 1), 1, wl.hkv, wl.d))
    if n:
        p = torch.from_numpy(idx_row[valid].astype(np.int64)).to(inp.q.device)
        pages = bt[p // wl.page].long()
        kc[:n, 0] = inp.k_cache[pages, p % wl.page].double().cpu().numpy()
        vc[:n, 0] = inp.v_cache[pages, p % wl.page].double().cpu().numpy()
    local = np.full(len(idx_row), -1, np.int64)
    local[valid] = np.arange(n)
    q = inp.q[r].double().cpu().numpy()
    po, pl = O.attention_split_row(q, kc, vc, np.arange(max(n, 1)), 1, local, wl.attn_scale, S)
    return po, pl, *O.merge_row(po, pl)


@pytest.mark.parametrize("S", [1, 2, 4, 8])
def test_attention_padding_anywhere(S):
    """Selections with -1 runs at the start of a split, in its middle, and
    whole empty splits: padding slots weigh nothing, nothing turns NaN, and
    partials (two launches) and outputs (fused) match the oracle."""
    from sparse_attention_decode_02_amd import lib
    _say(f"attention with padding anywhere, splits {S}")
    step = run_step(_host_inputs(_small_mixed(seed=41)), num_splits=S)
    wl, inp = step.wl, step.inp
    gidx = _gapped_idx(step, np.random.default_rng(S))
    idx_d = torch.from_numpy(gidx).cuda()
    po = torch.empty_like(step.part_o)
    pl = torch.empty_like(step.part_lse)
    lib.sparse_attn(inp.q, inp.k_cache, inp.v_cache, inp.block_table, step.row_req, idx_d,
                    wl.page, wl.attn_scale, S, po, pl)
    out = torch.empty_like(step.out)
    out_lse = torch.empty_like(step.out_lse)
    lib.sparse_attn_merged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, step.row_req, idx_d,
                           wl.page, wl.attn_scale, S, out, out_lse)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(po).any()) and not bool(torch.isnan(out.float()).any())
    tol_o, tol_l = 2e-2, 1e-3
    for r in range(step.rows):
        wpo, wpl, wo, wl_ = _oracle_attention(step, r, gidx[r], S)
        gpl = pl[r].double().cpu().numpy()
        assert np.array_equal(np.isfinite(gpl), np.isfinite(wpl)), r
        fin = np.isfinite(wpl)
        if fin.any():
            assert float(np.abs(gpl[fin] - wpl[fin]).max()) <= tol_l, r
        assert float(np.abs(po[r].double().cpu().numpy() - wpo).max()) <= tol_o, r
        assert float(np.abs(out[r].double().cpu().numpy() - wo).max()) <= tol_o, r
        gl = out_lse[r].double().cpu().numpy()
        assert np.array_equal(np.isfinite(gl), np.isfinite(wl_)), r
        fl = np.isfinite(wl_)
        if fl.any():
            assert float(np.abs(gl[fl] - wl_[fl]).max()) <= tol_l, r


def _prefill_groups_wl(seed=51, topk=256, page=64):
    # Prefill chunks of 37, 9, 8 and 3 rows on short and long prior contexts
    # (unions spanning several of the kernel's 1024-position windows), plus
    # two decode rows; 64 query / 8 KV heads of dim 128 (8 heads per group).
    prior = (700, 5000, 60, 0, 20000, 3000, 9)
    new = (37, 9, 8, 3, 6, 1, 1)
    return I.custom(I.decode(), name="prefill_groups", hq=64, hkv=8, topk=topk, prior=prior,
                    new=new, seed=seed, page=page)


@pytest.mark.parametrize("block_rows,topk,page", [(8, 256, 64), (3, 256, 64), (8, 2048, 64),
                                                  (1, 64, 64), (8, 256, 16), (5, 2048, 128)])
def test_group_attn_matches_oracle(block_rows, topk, page):
    """dsa_group_attn (the union of a group's selections with per-row masks,
    matrix cores) writes every row's attention output and log-sum-exp within
    the bf16 tolerances of the oracle, for groups of 1..8 rows and pages of
    16, 64 and 128 positions (each union entry's cache row comes through the
    block table)."""
    from sparse_attention_decode_02_amd import lib
    inp = _host_inputs(_prefill_groups_wl(topk=topk, page=page))
    step = run_step(inp, block_rows=1, num_splits=1)
    groups_host = lib.plan_blocks(step.row_req_host, block_rows)
    groups = torch.from_numpy(groups_host).cuda()
    wl = step.wl
    out = torch.full_like(step.out, float("nan"))
    lse = torch.full_like(step.out_lse, float("nan"))
    lib.group_attn(inp.q, inp.k_cache, inp.v_cache, inp.block_table, step.row_req, step.idx,
                   groups, wl.page, wl.attn_scale, out, lse)
    torch.cuda.synchronize()
    _say(f"group attention: {step.rows} rows in {len(groups_host)} groups of <= {block_rows}")
    worst = 0.0
    for r in range(step.rows):
        _, idx, _, _, o, ol = oracle_row(step, r)
        assert np.array_equal(step.idx[r].cpu().numpy(), idx)
        go = out[r].double().cpu().numpy()
        gl = lse[r].double().cpu().numpy()
        err = float(np.abs(go - o).max())
        worst = max(worst, err)
        assert err <= 2e-2, f"row {r}: output error {err}"
        fin = np.isfinite(ol)
        assert np.array_equal(np.isfinite(gl), fin), r
        if fin.any():
            assert float(np.abs(gl[fin] - ol[fin]).max()) <= 1e-3, f"row {r}: lse"
    _say(f"  max |out err| {worst:.3g}")


def test_group_attn_step():
    """The step with prefill groups on the matrix cores and the trailing
    decode rows on the split attention kernel: every row against the oracle."""
    inp = _host_inputs(_prefill_groups_wl(seed=53))
    step = DsaStep(inp, block_rows=8, fused=None, group_attn=True)
    step.scores.view(torch.int32).fill_(CANARY)
    step.run()
    torch.cuda.synchronize()
    assert step.groups is not None and step.group_rows < step.rows
    for r in range(step.rows):
        _, idx, _, _, o, ol = oracle_row(step, r)
        assert np.array_equal(step.idx[r].cpu().numpy(), idx)
        assert float(np.abs(step.out[r].double().cpu().numpy() - o).max()) <= 2e-2, r


def test_group_attn_automatic_choice():
    """group_attn=None: on where the blocks' rows are short against top-k
    (same bits as group_attn=True), off where they are long (same bits as
    the split attention kernel)."""
    short = I.custom(I.decode(), name="prefill_groups_short", hq=64, hkv=8, topk=2048,
                     prior=(700, 5000, 60, 0, 3000, 9), new=(37, 9, 8, 3, 1, 1), seed=55)
    inp = _host_inputs(short)
    auto = run_step(inp, block_rows=8, fused=None, group_attn=None)
    on = run_step(inp, block_rows=8, fused=None, group_attn=True)
    assert auto.groups is not None
    assert torch.equal(auto.out.view(torch.int16), on.out.view(torch.int16))
    for r in (0, 36, 40, auto.rows - 1):
        _, _, _, _, o, _ = oracle_row(auto, r)
        assert float(np.abs(auto.out[r].double().cpu().numpy() - o).max()) <= 2e-2, r
    inp = _host_inputs(_prefill_groups_wl(seed=54, topk=256))  # rows up to 20006 > 8 x 256
    auto = run_step(inp, block_rows=8, fused=None, group_attn=None)
    off = run_step(inp, block_rows=8, fused=None, group_attn=False)
    assert auto.groups is None
    assert torch.equal(auto.out.view(torch.int16), off.out.view(torch.int16))


def test_group_attn_zero_length_rows():
    """Rows of length 0 inside a group select nothing: output 0, lse -inf,
    and the group's other rows are unaffected."""
    from sparse_attention_decode_02_amd import lib
    inp = _host_inputs(_prefill_groups_wl(seed=52))
    step = run_step(inp, block_rows=1, num_splits=1)
    pad = [3, 10, 40]
    step.row_len[pad] = 0
    step.run()
    torch.cuda.synchronize()
    step.row_len_host = step.row_len.cpu().numpy()
    groups = torch.from_numpy(lib.plan_blocks(step.row_req_host, 8)).cuda()
    wl = step.wl
    out = torch.full_like(step.out, float("nan"))
    lse = torch.full_like(step.out_lse, float("nan"))
    lib.group_attn(inp.q, inp.k_cache, inp.v_cache, inp.block_table, step.row_req, step.idx,
                   groups, wl.page, wl.attn_scale, out, lse)
    torch.cuda.synchronize()
    for r in pad:
        assert bool((out[r].float() == 0).all()) and bool(torch.isneginf(lse[r]).all())
    for r in (0, 2, 4, 9, 11, 39, 41):
        _, _, _, _, o, ol = oracle_row(step, r)
        assert float(np.abs(out[r].double().cpu().numpy() - o).max()) <= 2e-2, r


def test_padding_rows_with_zero_length():
    """Rows of length 0 (padding in a fixed-size batch): no score written, all
    slots -1, empty attention (o = 0, lse = -inf), merged output 0."""
    wl = _small_mixed(seed=3)
    step = run_step(_host_inputs(wl), num_splits=4)
    pad = [2, 40, step.rows - 1]
    step.row_len[pad] = 0
    step.scores.view(torch.int32).fill_(CANARY)
    step.run()
    torch.cuda.synchronize()
    for r in pad:
        assert bool((step.scores[r].view(torch.int32) == CANARY).all())
        assert bool((step.idx[r] == -1).all())
        assert bool(torch.isneginf(step.part_lse[r]).all())
        assert bool((step.part_o[r] == 0).all())
        assert bool((step.out[r].float() == 0).all())
        assert bool(torch.isneginf(step.out_lse[r]).all())
    # the other rows are unaffected
    step.row_len_host = step.row_len.cpu().numpy()
    for r in (0, 41):
        check_row(step, r)


def test_score_blocks_are_bit_identical():
    wl = _small_mixed(seed=9)
    inp = _host_inputs(wl)
    ref = run_step(inp, block_rows=1).scores.clone()
    for br in (2, 5, 16, 64):
        s = run_step(inp, block_rows=br).scores
        assert torch.equal(s.view(torch.int32), ref.view(torch.int32)), f"block_rows {br}"


def test_score_blocks_fp32_bit_identical():
    """fp32 inputs with prefill rows in score blocks (the fp32 kernel scores a
    block's rows one after another): the same bits as one row per block, and
    every row against the oracle."""
    wl = I.custom(I.tiny(), name="tiny_prefill_fp32", prior=(30, 90, 0), new=(7, 10, 5), seed=17)
    inp = _host_inputs(wl)
    ref = run_step(inp, block_rows=1)
    for br in (2, 4, 16):
        st = run_step(inp, block_rows=br)
        assert len(st.blocks_host) < st.rows
        assert torch.equal(st.scores.view(torch.int32), ref.scores.view(torch.int32)), f"block_rows {br}"
        assert torch.equal(st.idx, ref.idx)
    e = _check_all(ref)
    _say(f"fp32 score blocks, {ref.rows} rows: max errors {e}")


def _block_mix(hi, di, page, seed=31):
    # Blocks of 37 (8+8+8+8+5 rows), 16, 9 (8+1) and 64 rows, and of 2, 3, 6,
    # 7 rows (4, 2, 1, 1 waves per row) for the block kernel, and one block
    # of one row for the row kernel launched beside it: 145 rows in 9 blocks.
    # Lengths cross tiles, stages, pages and chunks.
    prior = (0, 130, 1000, 5000, 62, 255, 2999, 16, 700)
    new = (37, 16, 9, 64, 1, 2, 3, 6, 7)
    return I.custom(I.decode(), name=f"block_mix_{hi}x{di}_p{page}", hq=16, hkv=2, hi=hi, di=di,
                    page=page, topk=256, prior=prior, new=new, seed=seed)


@pytest.mark.parametrize("hi,di,page", [(64, 128, 64), (32, 128, 16), (64, 64, 16), (32, 64, 64)])
def test_block_indexer_matches_row_kernel(hi, di, page):
    """Scores of score blocks (query blocks in registers, keys shared
    through LDS) equal the one-row-per-block scores bit for bit, unwritten
    positions included; rows of length 0 inside a block stay unwritten."""
    inp = _host_inputs(_block_mix(hi, di, page))
    ref = run_step(inp, block_rows=1)
    blk = run_step(inp, block_rows=64)
    _say(f"indexer {hi}x{di}, page {page}: {blk.rows} rows in {len(blk.blocks_host)} blocks")
    assert torch.equal(blk.scores.view(torch.int32), ref.scores.view(torch.int32))
    assert torch.equal(blk.idx, ref.idx)
    if (hi, di, page) == (64, 128, 64):
        _check_all(blk)
    pad = [3, 40, 53, 100]  # inside the 37-, 16-, 9- and 64-row blocks
    for st in (ref, blk):
        st.row_len[pad] = 0
        st.scores.view(torch.int32).fill_(CANARY)
        st.run()
    torch.cuda.synchronize()
    assert torch.equal(blk.scores.view(torch.int32), ref.scores.view(torch.int32))
    for r in pad:
        assert bool((blk.scores[r].view(torch.int32) == CANARY).all())


@pytest.mark.parametrize("block_rows", [1, 8], ids=["rows", "blocks"])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "two-launch"])
def test_graph_replay_matches_eager(fused, block_rows):
    """The step recorded into a HIP graph and replayed gives the eager step's
    bits on every replay, with eager work in between, and follows row lengths
    changed in device memory between replays (same width). With score blocks
    the block and row indexer kernels run on two streams, forked and joined
    inside the recording."""
    _say(f"graph replay, fused {fused}, block_rows {block_rows}")
    inp = _host_inputs(_small_mixed(seed=17))
    step = DsaStep(inp, num_splits=4, fused=fused, block_rows=block_rows)
    outs = lambda: [t.clone() for t in (step.scores, step.idx, step.out, step.out_lse)]

    def same(a, b):
        # scores past a row's length are not written: compare the written part
        la = step.row_len.cpu().numpy()
        for r in range(step.rows):
            assert torch.equal(a[0][r, : la[r]].view(torch.int32), b[0][r, : la[r]].view(torch.int32)), r
        for x, y in zip(a[1:], b[1:]):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))

    def clear():
        step.scores.view(torch.int32).fill_(CANARY)
        for t in (step.idx, step.out, step.out_lse):
            t.zero_()

    clear()
    step.run()
    torch.cuda.synchronize()
    eager = outs()
    graph = step.capture()
    torch.cuda.synchronize()
    other = DsaStep(_host_inputs(_small_mixed(seed=18)), num_splits=2)
    for rep in range(3):
        clear()
        graph.replay()
        torch.cuda.synchronize()
        same(outs(), eager)
        other.run()  # eager work between replays
        torch.cuda.synchronize()
    # shorter rows in place, then eager and replayed results must agree
    new_len = step.row_len.clone()
    new_len[::3] = torch.clamp(new_len[::3] - 37, min=0)
    step.row_len.copy_(new_len)
    clear()
    step.run()
    torch.cuda.synchronize()
    eager2 = outs()
    for rep in range(2):
        clear()
        graph.replay()
        torch.cuda.synchronize()
        same(outs(), eager2)
    step.row_len_host = new_len.cpu().numpy()
    for r in (0, 3, 36, step.rows - 1):
        check_row(step, r)


def _ragged_rows(seed=43):
    """Twelve decode rows from 1 to 40001 keys: many 1024-key chunks, unevenly."""
    prior = (40000, 0, 300, 9000, 25000, 4095, 17, 12000, 1023, 1024, 30000, 6)
    return I.custom(I.decode(), name="ragged_rows", hq=16, hkv=2, topk=256, prior=prior,
                    new=(1,) * len(prior), seed=seed)


@pytest.mark.parametrize("wl_fn", [I.decode, lambda: _small_mixed(seed=31), _ragged_rows],
                         ids=["decode", "small-mixed", "ragged"])
def test_indexer_hint_keeps_scores(wl_fn):
    """The total-keys hint (larger key chunks for rows that fill the width;
    for ragged one-row batches, a grid of about one workgroup per active
    chunk, balanced over the XCDs) changes the launch shape, never a score
    bit: a hint below the true count makes workgroups take several chunks."""
    from sparse_attention_decode_02_amd import lib
    step = run_step(_host_inputs(wl_fn()))
    i = step.inp
    ref = step.scores.clone()
    for total in (0, 1, step.total_keys // 3, step.total_keys, step.rows * step.width):
        step.scores.view(torch.int32).fill_(CANARY)
        lib.indexer_scores(i.qI, i.w, i.kI_cache, i.block_table, step.row_req, step.row_len,
                           step.scores, step.wl.page, total_keys=total)
        torch.cuda.synchronize()
        assert torch.equal(step.scores.view(torch.int32), ref.view(torch.int32)), total


def test_read_probe_reads_every_word():
    """The streaming-read probe of the benchmark sums every 16-byte word once."""
    from sparse_attention_decode_02_amd import lib
    x = torch.ones((64 << 20) // 4, dtype=torch.float32, device="cuda")
    x[-4:] = 3.0  # the tail is read too
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    lib.read_probe(x, sink)
    torch.cuda.synchronize()
    assert float(sink.double().sum()) == x.numel() + 8


def test_determinism():
    inp = _host_inputs(I.decode())
    a = run_step(inp)
    outs = [t.clone() for t in (a.scores, a.idx, a.part_o, a.part_lse, a.out, a.out_lse)]
    b = run_step(inp)
    for x, y in zip(outs, (b.scores, b.idx, b.part_o, b.part_lse, b.out, b.out_lse)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


# --------------------------------------------------------------------------
# Full-size workloads (the benchmark's launch configuration), sampled rows
# --------------------------------------------------------------------------


def _same_selection_other_ways(step):
    """At full size, the two-stage top-k and the windowed indexer + top-k
    reproduce the step's indices bit for bit."""
    from sparse_attention_decode_02_amd import lib
    wl, inp = step.wl, step.inp
    chunk = max(wl.topk, 8192)
    cand = torch.empty(lib.topk_chunked_slots(step.rows, step.width, wl.topk, chunk),
                       dtype=torch.int32, device="cuda")
    idx = torch.full_like(step.idx, -7)
    lib.topk_chunked(step.scores, step.row_len, wl.topk, chunk, cand, idx)
    torch.cuda.synchronize()
    assert torch.equal(idx, step.idx), "two-stage top-k differs"
    del cand
    # Windows of 16 rows over the step's score blocks (at most 8 rows each).
    window = 16
    buf = torch.empty(window * step.width, dtype=torch.float32, device="cuda")
    idx.fill_(-7)
    lib.indexer_topk_windowed(inp.qI, inp.w, inp.kI_cache, inp.block_table, step.row_req,
                              step.row_len, step.width, wl.page, wl.topk, buf, idx,
                              blocks=step.blocks, blocks_host=step.blocks_host)
    torch.cuda.synchronize()
    assert torch.equal(idx, step.idx), "windowed indexer + top-k differs"
    del buf
    # The histogram path: the indexer again (same scores, now with each row's
    # counts), then the selection from the counts.
    hist = torch.zeros(step.rows, lib.HIST_BINS, dtype=torch.int32, device="cuda")
    ref_scores_sum = float(step.scores[0, : int(step.row_len_host[0])].double().sum())
    lib.indexer_scores_hist(inp.qI, inp.w, inp.kI_cache, inp.block_table, step.row_req,
                            step.row_len, step.scores, hist, wl.page, blocks=step.blocks,
                            total_keys=step.total_keys)
    torch.cuda.synchronize()
    assert float(step.scores[0, : int(step.row_len_host[0])].double().sum()) == ref_scores_sum
    assert torch.equal(hist.sum(1, dtype=torch.int64), step.row_len.long()), "histogram counts"
    idx.fill_(-7)
    lib.topk_hist(step.scores, step.row_len, hist, wl.topk, idx, total_keys=step.total_keys)
    torch.cuda.synchronize()
    assert torch.equal(idx, step.idx), "histogram top-k differs"
    assert not bool(hist.any())
    _say(f"  two-stage top-k (chunk {chunk}), {window}-row windows and the histogram path: "
         "identical indices")


def _full(wl, rows_fn):
    _say(f"{wl.name}: generating on the device")
    inp = I.generate(wl, "cuda")
    # bench.py's launch configuration, with the one-pass or two-stage top-k;
    # the histogram top-k it may take instead must give the same indices
    # (checked in _same_selection_other_ways).
    step = run_step(inp, fused=None, block_rows=8)
    _say(f"  rows {step.rows}, width {step.width}, splits {step.num_splits}")
    check_properties(step)
    _same_selection_other_ways(step)
    rows = rows_fn(step)
    errs = {}
    for i, r in enumerate(rows):
        e = check_row(step, r)
        errs = {k: max(errs.get(k, 0.0), v) for k, v in e.items()}
        if i % 16 == 15 or i == len(rows) - 1:
            _say(f"  {i + 1}/{len(rows)} rows ok (last: row {r}, L={int(step.row_len_host[r])})")
    _say(f"  max errors {errs}")
    del step, inp
    torch.cuda.empty_cache()


def test_headline_full_size():
    """Every row of the batch-64, 32K-context decode against the oracle."""
    _full(I.headline(), lambda s: list(range(s.rows)))


def test_prefill_1m_full_size():
    """A 2048-token prefill chunk at 1M context (8 GiB of scores at once), in
    the bench's configuration, then checked as every full-size workload is."""
    _full(I.prefill_1m(), lambda s: [0, s.rows - 1])


def test_long_context_full_size():
    _full(I.long_context(), lambda s: [0, s.rows - 1])


def test_ragged_full_size():
    """Every row of the ragged batch (lengths 1 .. 65536) against the oracle."""
    def rows(s):
        L = s.row_len_host
        assert int(L.min()) == 1 and int(L.max()) == 65536
        assert any(1 < x < 2048 for x in L)
        return list(range(s.rows))
    _full(I.ragged(), rows)


def test_mixed_group_attn_full_size():
    """The mixed step with its prefill groups on the matrix cores (union of
    each 8-row group's selections) and its decode rows on the split attention
    kernel:
    sampled prefill rows, including each request's first and last, and decode
    rows against the oracle."""
    wl = I.mixed()
    _say(f"{wl.name} with group attention: generating on the device")
    inp = I.generate(wl, "cuda")
    step = DsaStep(inp, block_rows=8, fused=None, group_attn=True)
    step.scores.view(torch.int32).fill_(CANARY)
    step.run()
    torch.cuda.synchronize()
    assert step.group_rows == 2048
    rows = sorted({0, 7, 8, 63, 511, 512, 1023, 1024, 1535, 1536, 2047, 2048, 2080, 2107})
    errs = {}
    for r in rows:
        e = check_row(step, r)
        errs = {k: max(errs.get(k, 0.0), v) for k, v in e.items()}
    _say(f"  {len(rows)} rows ok, max errors {errs}")
    del step, inp
    torch.cuda.empty_cache()


def test_mixed_full_size():
    """All 60 decode rows, every 64th prefill row and the last row of each
    prefill request against the oracle."""
    def rows(s):
        n_pre = int(sum(n for n in s.wl.new if n > 1))
        assert n_pre == 2048 and s.rows == 2108
        pre = set(range(0, n_pre, 64)) | {511, 512, 1023, 1535, 2047}
        return sorted(pre | set(range(n_pre, s.rows)))
    _full(I.mixed(), rows)
