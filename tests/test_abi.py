"""CPU tests of the C ABI: the library loads without a GPU, exports every
symbol include/dsa.h declares, plans rows exactly as the oracle does, and
rejects every invalid host argument with its status code before any launch.
No test here enqueues GPU work: every kernel entry point is called only with
arguments it must reject (or with zero rows, which returns before launching).
"""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import dsa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

lib = pytest.importorskip("sparse_attention_decode_02_amd.lib",
                          reason="libdsa.so not built (python -m sparse_attention_decode_02_amd.build)")

OK, NULL, SHAPE, ALIGN, UNSUP, WS = 0, -1, -2, -3, -4, -5


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "dsa.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(dsa_\w+)\(", hdr, re.M))
    assert {"dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn", "dsa_merge"} <= declared
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name
    assert declared == set(lib.EXPORTS)


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert lib.status_string(s) and lib.status_string(s) != "unknown status"
    assert lib.status_string(-99) == "unknown status"
    assert lib.abi_version() >= 1


# --------------------------------------------------------------------------
# Row plan: bit-exact with the oracle
# --------------------------------------------------------------------------


def test_plan_rows_matches_oracle(golden):
    g = golden["row_plan"]
    req, ln = lib.plan_rows(g["prior"], g["new"])
    assert req.tolist() == g["row_req"] and ln.tolist() == g["row_len"]
    rng = np.random.default_rng(0)
    for _ in range(50):
        n = int(rng.integers(0, 12))
        prior = rng.integers(0, 10000, n)
        new = rng.integers(0, 40, n)
        a = lib.plan_rows(prior, new)
        b = O.row_plan(prior, new)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_plan_blocks_matches_oracle():
    rng = np.random.default_rng(1)
    for _ in range(50):
        req = np.sort(rng.integers(0, 6, int(rng.integers(1, 60)))).astype(np.int32)
        for m in (1, 2, 5, 16, 128):
            assert np.array_equal(lib.plan_blocks(req, m), O.score_blocks(req, m))


def test_group_attention_automatic_choice():
    """The step takes group attention when it has blocks of 2..8 rows and none
    of their rows is longer than 8 x top-k (host logic; no launches)."""
    from sparse_attention_decode_02_amd.step import group_attention_pays
    # 4 prefill rows on a 1000-key prior context, then 2 decode rows
    req, ln = lib.plan_rows(np.array([1000, 9000, 50], np.int32), np.array([4, 1, 1], np.int32))
    blocks = lib.plan_blocks(req, 8)
    assert group_attention_pays(blocks, ln, 2048, 8)          # longest block row 1004
    assert not group_attention_pays(blocks, ln, 100, 8)       # 1004 > 800
    assert not group_attention_pays(None, ln, 2048, 1)        # no blocks
    assert not group_attention_pays(blocks, ln, 2048, 16)     # blocks wider than a group
    one = lib.plan_blocks(req, 1)                             # only one-row blocks
    assert not group_attention_pays(one, ln, 2048, 1)
    # a long decode row does not count: only rows of multi-row blocks do
    req2, ln2 = lib.plan_rows(np.array([100, 900000], np.int32), np.array([8, 1], np.int32))
    assert group_attention_pays(lib.plan_blocks(req2, 8), ln2, 2048, 8)


def test_histogram_topk_automatic_choice():
    """The step takes the histogram top-k when it selects in one pass, has no
    multi-row score blocks and some row is longer than the one-pass kernel
    holds at 32 keys per thread; with multi-row blocks, only when some of
    their rows is longer than the one-pass kernel holds at all (host logic;
    no launches)."""
    from sparse_attention_decode_02_amd.step import ONE_PASS_RESIDENT_KEYS, histogram_topk_pays
    assert ONE_PASS_RESIDENT_KEYS == 32768
    req, ln = lib.plan_rows(np.array([65535, 2000, 40], np.int32), np.array([1, 1, 1], np.int32))
    assert histogram_topk_pays(None, ln, True)                       # a 65536-key decode row
    assert histogram_topk_pays(lib.plan_blocks(req, 8), ln, True)    # one-row blocks only
    assert not histogram_topk_pays(None, ln, False)                  # two stages or windows
    req2, ln2 = lib.plan_rows(np.array([32767] * 3, np.int32), np.array([1] * 3, np.int32))
    assert not histogram_topk_pays(None, ln2, True)                  # 32768 keys fit one pass
    req3, ln3 = lib.plan_rows(np.array([65535, 100], np.int32), np.array([1, 4], np.int32))
    assert not histogram_topk_pays(lib.plan_blocks(req3, 8), ln3, True)  # a prefill block
    assert histogram_topk_pays(lib.plan_blocks(req3, 1), ln3, True)      # rows scored alone
    assert not histogram_topk_pays(None, ln[:0], True)               # no rows
    # prefill blocks of rows beyond 65536 keys (two-stage territory)
    req4, ln4 = lib.plan_rows(np.array([65533, 200], np.int32), np.array([4, 1], np.int32))
    assert int(ln4[:4].max()) == 65537
    assert histogram_topk_pays(lib.plan_blocks(req4, 8), ln4, False)
    assert histogram_topk_pays(lib.plan_blocks(req4, 8), ln4, True)
    req5, ln5 = lib.plan_rows(np.array([65532], np.int32), np.array([4], np.int32))
    assert int(ln5.max()) == 65536
    assert not histogram_topk_pays(lib.plan_blocks(req5, 8), ln5, False)  # fits one pass


def test_score_width():
    assert lib.score_width([37, 100]) == 128
    assert lib.score_width([64]) == 64
    assert lib.score_width([65]) == 128
    assert lib.score_width([1]) == 64
    assert lib.score_width([32768] * 3) == 32768


def test_plan_errors():
    nr = ctypes.c_int(0)
    p = np.asarray([1, 2], np.int32)
    n = np.asarray([1, -1], np.int32)
    out = np.zeros(4, np.int32)
    assert lib._lib.dsa_plan_rows(2, p.ctypes.data, n.ctypes.data, 4, out.ctypes.data,
                                  out.ctypes.data, ctypes.byref(nr)) == SHAPE
    n = np.asarray([3, 3], np.int32)
    assert lib._lib.dsa_plan_rows(2, p.ctypes.data, n.ctypes.data, 4, out.ctypes.data,
                                  out.ctypes.data, ctypes.byref(nr)) == SHAPE  # 6 rows > 4
    assert lib._lib.dsa_plan_rows(2, None, n.ctypes.data, 8, out.ctypes.data, out.ctypes.data,
                                  ctypes.byref(nr)) == NULL
    big = np.asarray([2**31 - 1], np.int32)
    one = np.asarray([1], np.int32)
    assert lib._lib.dsa_plan_rows(1, big.ctypes.data, one.ctypes.data, 4, out.ctypes.data,
                                  out.ctypes.data, ctypes.byref(nr)) == SHAPE
    req = np.asarray([0, 1, 2], np.int32)
    bl = np.zeros((2, 2), np.int32)
    assert lib._lib.dsa_plan_blocks(3, req.ctypes.data, 1, 2, bl.ctypes.data, ctypes.byref(nr)) == SHAPE
    assert lib._lib.dsa_plan_blocks(3, req.ctypes.data, 0, 4, bl.ctypes.data, ctypes.byref(nr)) == SHAPE
    assert lib._lib.dsa_score_width(1, np.asarray([-1], np.int32).ctypes.data, ctypes.byref(nr)) == SHAPE


# --------------------------------------------------------------------------
# Kernel entry points: argument checks (no launch)
# --------------------------------------------------------------------------

A = 1 << 20  # a fake 16-byte-aligned device address; never dereferenced


def _indexer_args(**kw):
    a = dict(q_idx=A, w=A, k_idx_cache=A, block_table=A, row_req=A, row_len=A, blocks=None,
             num_blocks=0, scores=A, rows=4, width=128, num_heads=64, head_dim=128, page_size=64,
             max_pages=8, dtype=1, stream=None)
    a.update(kw)
    return list(a.values())


def _topk_args(**kw):
    a = dict(scores=A, row_len=A, rows=4, width=128, k=16, idx=A, stream=None)
    a.update(kw)
    return list(a.values())


def _attn_args(**kw):
    a = dict(q=A, k_cache=A, v_cache=A, block_table=A, row_req=A, idx=A, rows=4, hq=64, hkv=8,
             d=128, k=2048, page_size=64, max_pages=8, scale=0.088, num_splits=8, part_o=A,
             part_lse=A, dtype=1, stream=None)
    a.update(kw)
    return list(a.values())


def _merge_args(**kw):
    a = dict(part_o=A, part_lse=A, rows=4, hq=64, d=128, num_splits=8, out=A, out_lse=A,
             dtype=1, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q_idx=None), NULL), (dict(w=None), NULL), (dict(k_idx_cache=None), NULL),
    (dict(block_table=None), NULL), (dict(row_req=None), NULL), (dict(row_len=None), NULL),
    (dict(scores=None), NULL),
    (dict(rows=-1), SHAPE), (dict(width=0), SHAPE), (dict(width=130), SHAPE),
    (dict(max_pages=0), SHAPE), (dict(page_size=48), SHAPE), (dict(page_size=0), SHAPE),
    (dict(blocks=A, num_blocks=0), SHAPE), (dict(blocks=A, num_blocks=5), SHAPE),
    (dict(num_heads=48), UNSUP), (dict(head_dim=96), UNSUP), (dict(dtype=7), UNSUP),
    (dict(page_size=8), UNSUP), (dict(page_size=8, dtype=0, num_heads=4, head_dim=32, scores=A + 4), ALIGN),
    (dict(dtype=0, num_heads=65), UNSUP), (dict(dtype=0, head_dim=256), UNSUP),
    (dict(q_idx=A + 2), ALIGN), (dict(k_idx_cache=A + 8), ALIGN), (dict(scores=A + 4), ALIGN),
    (dict(w=A + 2), ALIGN), (dict(blocks=A + 2, num_blocks=2), ALIGN),
    (dict(rows=0), OK),
])
def test_indexer_rejects(kw, code):
    assert lib._lib.dsa_indexer_scores(*_indexer_args(**kw)) == code


@pytest.mark.parametrize("total,kw,code", [
    (-1, {}, SHAPE), (4 * 128 + 1, {}, SHAPE), (4 * 128, dict(q_idx=None), NULL),
    (4 * 128, dict(width=130), SHAPE), (0, dict(rows=0), OK), (4 * 128, dict(rows=0), SHAPE),
])
def test_indexer_total_rejects(total, kw, code):
    args = _indexer_args(**kw)
    assert lib._lib.dsa_indexer_scores_total(*args[:-1], total, args[-1]) == code


@pytest.mark.parametrize("kw,code", [
    (dict(scores=None), NULL), (dict(row_len=None), NULL), (dict(idx=None), NULL),
    (dict(rows=-1), SHAPE), (dict(width=0), SHAPE), (dict(width=66), SHAPE), (dict(k=0), SHAPE),
    (dict(k=129), SHAPE), (dict(scores=A + 4), ALIGN), (dict(idx=A + 1), ALIGN),
    (dict(rows=0), OK),
])
def test_topk_rejects(kw, code):
    assert lib._lib.dsa_topk(*_topk_args(**kw)) == code


@pytest.mark.parametrize("total,kw,code", [
    (-1, {}, SHAPE), (4 * 128 + 1, {}, SHAPE), (4 * 128, dict(scores=None), NULL),
    (4 * 128, dict(width=66), SHAPE), (0, dict(rows=0), OK), (4 * 128, dict(rows=0), SHAPE),
    (4 * 128, dict(idx=A + 1), ALIGN),
])
def test_topk_total_rejects(total, kw, code):
    args = _topk_args(**kw)
    assert lib._lib.dsa_topk_total(*args[:-2], total, *args[-2:]) == code


def _chunked_args(**kw):
    a = dict(scores=A, row_len=A, rows=4, width=128, k=16, chunk=32, cand=A, cand_slots=2 * 4 * 4 * 16,
             idx=A, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(scores=None), NULL), (dict(cand=None), NULL), (dict(idx=None), NULL),
    (dict(chunk=8), SHAPE), (dict(chunk=30), SHAPE), (dict(chunk=(1 << 20) + 4, width=(1 << 20) + 64), SHAPE),
    (dict(k=0), SHAPE), (dict(width=66), SHAPE), (dict(cand_slots=2 * 4 * 4 * 16 - 1), WS),
    (dict(cand=A + 2), ALIGN), (dict(scores=A + 4), ALIGN), (dict(rows=0), OK),
])
def test_topk_chunked_rejects(kw, code):
    assert lib._lib.dsa_topk_chunked(*_chunked_args(**kw)) == code


def _noalloc_args(**kw):
    a = dict(scores=A, row_len=A, rows=4, width=128, k=16, chunk=32, idx=A, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(scores=None), NULL), (dict(row_len=None), NULL), (dict(idx=None), NULL),
    (dict(chunk=8), SHAPE), (dict(chunk=30), SHAPE), (dict(k=0), SHAPE), (dict(width=66), SHAPE),
    (dict(scores=A + 4), ALIGN), (dict(rows=0), OK),
    # 2 * rows * segments * k > DSA_TOPK_NOALLOC_MAX_SLOTS (1 << 22)
    (dict(rows=2048, width=4096, k=2048, chunk=2048), WS),
    (dict(rows=1025, width=4096, k=2048, chunk=4096), WS),
])
def test_topk_chunked_noalloc_rejects(kw, code):
    """Every status of the allocation-free call but a launch is decided on the
    host: oversized inputs are refused before the workspace is looked up."""
    assert lib._lib.dsa_topk_chunked_noalloc(*_noalloc_args(**kw)) == code


def test_topk_chunked_noalloc_limit():
    assert lib.TOPK_NOALLOC_MAX_SLOTS == 1 << 22
    assert lib.topk_chunked_slots(1024, 4096, 2048, 4096) == 1 << 22  # exactly fits
    assert lib.topk_chunked_slots(64, 204800, 2048, 32768) <= lib.TOPK_NOALLOC_MAX_SLOTS


def _topk_hist_args(**kw):
    a = dict(scores=A, row_len=A, hist=A, rows=4, width=128, k=16, total=0, idx=A, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(hist=None), NULL), (dict(scores=None), NULL), (dict(idx=None), NULL),
    (dict(hist=A + 4), ALIGN), (dict(k=0), SHAPE), (dict(k=129), SHAPE), (dict(width=66), SHAPE),
    (dict(total=-1), SHAPE), (dict(total=4 * 128 + 1), SHAPE), (dict(rows=0), OK),
])
def test_topk_hist_rejects(kw, code):
    assert lib._lib.dsa_topk_hist(*_topk_hist_args(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(hist=None), NULL), (dict(scores=None), NULL), (dict(hist=A + 8), ALIGN),
    (dict(row_len=A + 2), ALIGN), (dict(rows=-1), SHAPE), (dict(width=0), SHAPE), (dict(rows=0), OK),
])
def test_score_hist_rejects(kw, code):
    a = dict(scores=A, row_len=A, rows=4, width=128, hist=A, stream=None)
    a.update(kw)
    assert lib._lib.dsa_score_hist(*a.values()) == code


@pytest.mark.parametrize("kw,code", [
    (dict(hist=None), NULL), (dict(hist=A + 4), ALIGN), (dict(total=-1), SHAPE),
    (dict(q_idx=None), NULL), (dict(head_dim=96), UNSUP), (dict(rows=0, total=0), OK),
])
def test_indexer_scores_hist_rejects(kw, code):
    a = dict(q_idx=A, w=A, k_idx_cache=A, block_table=A, row_req=A, row_len=A, blocks=None,
             num_blocks=0, scores=A, hist=A, rows=4, width=128, num_heads=64, head_dim=128,
             page_size=64, max_pages=2, dtype=1, total=0, stream=None)
    a.update(kw)
    assert lib._lib.dsa_indexer_scores_hist(*a.values()) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(groups=None), NULL), (dict(groups=None, num_groups=0), OK),
    (dict(num_groups=5), SHAPE), (dict(num_q_heads=63), SHAPE), (dict(page_size=48), SHAPE),
    (dict(head_dim=64), UNSUP), (dict(num_q_heads=32), UNSUP), (dict(dtype=0), UNSUP),
    (dict(k_cache=A + 8), ALIGN), (dict(rows=0, num_groups=0), OK),
])
def test_group_attn_rejects(kw, code):
    a = dict(q=A, k_cache=A, v_cache=A, block_table=A, row_req=A, idx=A, groups=A, num_groups=2,
             rows=4, num_q_heads=64, num_kv_heads=8, head_dim=128, k=16, page_size=64,
             max_pages=4, scale=0.1, out=A, out_lse=None, dtype=1, stream=None)
    a.update(kw)
    if kw.get("num_groups", 2) == 0 and code == OK:
        # accepted and nothing launched
        pass
    assert lib._lib.dsa_group_attn(*a.values()) == code


def test_topk_chunked_slots():
    assert lib.topk_chunked_slots(4, 128, 16, 32) == 2 * 4 * 4 * 16
    assert lib.topk_chunked_slots(4, 132, 16, 32) == 2 * 4 * 5 * 16
    assert lib.topk_chunked_slots(3, 32768, 2048, 8192) == 2 * 3 * 4 * 2048
    with pytest.raises(lib.DsaError):
        lib.topk_chunked_slots(4, 128, 16, 8)


@pytest.mark.parametrize("plan,code", [
    ([(0, 2), (2, 2)], OK), ([(0, 1), (1, 3)], WS), ([(0, 2), (3, 1)], SHAPE),
    ([(0, 2), (2, 1)], SHAPE), ([(0, 0), (0, 4)], SHAPE), ([(1, 3)], SHAPE),
])
def test_windowed_block_plan(plan, code):
    """A block plan must cover the rows in order; a block longer than the
    window (2 rows here) cannot be placed. Every status is decided on the
    host before any launch; a valid plan is shown by the next check failing
    instead (an unsupported head dim), so the fake pointers are never used."""
    import numpy as np
    bh = np.asarray(plan, np.int32)
    args = _windowed_args(blocks_host=bh.ctypes.data, blocks_dev=A, num_blocks=len(plan))
    st = lib._lib.dsa_indexer_topk_windowed(*args)
    if code == OK:
        args = _windowed_args(blocks_host=bh.ctypes.data, blocks_dev=A, num_blocks=len(plan),
                              head_dim=96)
        assert lib._lib.dsa_indexer_topk_windowed(*args) == UNSUP
    else:
        assert st == code


def test_topk_chunk_suggest():
    assert lib.topk_chunk_suggest(64, 32768, 2048, 64 * 32768) == 0  # rows fit a workgroup
    assert lib.topk_chunk_suggest(2048, 1 << 20, 2048, 2048 << 20) == 32768  # full long rows
    assert lib.topk_chunk_suggest(2048, 1 << 17, 2048, 2048 * 9000) == 0  # mostly short rows
    out = ctypes.c_int(0)
    assert lib._lib.dsa_topk_chunk_suggest(4, 128, 16, -1, ctypes.byref(out)) == SHAPE
    assert lib._lib.dsa_topk_chunk_suggest(4, 128, 16, 4 * 128 + 1, ctypes.byref(out)) == SHAPE


def test_select_window_rows():
    assert lib.select_window_rows(128, 128 * 4 * 3 + 5) == 3
    assert lib.select_window_rows(32768, 1 << 30) == 8192
    out = ctypes.c_int(0)
    assert lib._lib.dsa_select_window_rows(128, 511, ctypes.byref(out)) == WS
    assert lib._lib.dsa_select_window_rows(0, 100, ctypes.byref(out)) == SHAPE
    assert lib._lib.dsa_select_window_rows(128, 4096, None) == NULL


@pytest.mark.parametrize("args,code", [
    ((None, 64, A, 4), NULL), ((A, 64, None, 4), NULL), ((A, 8, A, 4), SHAPE), ((A, 72, A, 4), SHAPE),
    ((A, 64, A, 0), SHAPE), ((A + 4, 64, A, 4), ALIGN), ((A, 64, A + 2, 4), ALIGN),
])
def test_read_probe_rejects(args, code):
    assert lib._lib.dsa_read_probe(*args, None) == code


def _windowed_args(**kw):
    a = dict(q_idx=A, w=A, k_idx_cache=A, block_table=A, row_req=A, row_len=A, blocks_host=None,
             blocks_dev=None, num_blocks=0, rows=4, width=128,
             num_heads=64, head_dim=128, page_size=64, max_pages=8, dtype=1, k=16, score_buffer=A,
             score_buffer_bytes=128 * 4 * 2, topk_chunk=0, cand=None, cand_slots=0, idx=A,
             stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(score_buffer_bytes=511), WS), (dict(score_buffer=None), NULL), (dict(q_idx=None), NULL),
    (dict(idx=None), NULL), (dict(topk_chunk=-1), SHAPE), (dict(topk_chunk=32), NULL),
    (dict(topk_chunk=32, cand=A, cand_slots=2 * 2 * 4 * 16 - 1), WS), (dict(topk_chunk=8, cand=A, cand_slots=999), SHAPE),
    (dict(k=0), SHAPE), (dict(head_dim=96), UNSUP), (dict(score_buffer=A + 4), ALIGN),
    (dict(page_size=48), SHAPE), (dict(rows=-1), SHAPE), (dict(rows=0), OK),
    (dict(num_blocks=2), NULL), (dict(num_blocks=-1), SHAPE),
])
def test_windowed_rejects(kw, code):
    assert lib._lib.dsa_indexer_topk_windowed(*_windowed_args(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k_cache=None), NULL), (dict(v_cache=None), NULL),
    (dict(block_table=None), NULL), (dict(row_req=None), NULL), (dict(idx=None), NULL),
    (dict(part_o=None), NULL), (dict(part_lse=None), NULL),
    (dict(rows=-1), SHAPE), (dict(hq=0), SHAPE), (dict(hkv=0), SHAPE), (dict(hkv=3), SHAPE),
    (dict(k=0), SHAPE), (dict(max_pages=0), SHAPE), (dict(num_splits=0), SHAPE),
    (dict(num_splits=2049), SHAPE), (dict(page_size=100), SHAPE),
    (dict(scale=float("inf")), SHAPE), (dict(scale=float("nan")), SHAPE),
    (dict(d=96), UNSUP), (dict(hq=24, hkv=8), UNSUP), (dict(hq=64, hkv=2), UNSUP),
    (dict(dtype=5), UNSUP),
    (dict(q=A + 2), ALIGN), (dict(k_cache=A + 4), ALIGN), (dict(v_cache=A + 8), ALIGN),
    (dict(part_o=A + 4), ALIGN), (dict(part_lse=A + 2), ALIGN), (dict(idx=A + 2), ALIGN),
    (dict(rows=0), OK),
])
def test_sparse_attn_rejects(kw, code):
    args = _attn_args(**kw)
    assert lib._lib.dsa_sparse_attn(*args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(part_o=None), NULL), (dict(part_lse=None), NULL), (dict(out=None), NULL),
    (dict(rows=-1), SHAPE), (dict(hq=0), SHAPE), (dict(d=0), SHAPE), (dict(d=257), SHAPE),
    (dict(num_splits=0), SHAPE), (dict(dtype=3), UNSUP),
    (dict(part_o=A + 4), ALIGN), (dict(out=A + 2), ALIGN), (dict(out_lse=A + 2), ALIGN),
    (dict(part_lse=A + 1), ALIGN), (dict(rows=0), OK),
])
def test_merge_rejects(kw, code):
    assert lib._lib.dsa_merge(*_merge_args(**kw)) == code


@pytest.mark.parametrize("args,code", [
    ((4, 64, 8, 128, 2048, 1, None), NULL),
    ((0, 64, 8, 128, 2048, 1, "out"), SHAPE), ((4, 64, 0, 128, 2048, 1, "out"), SHAPE),
    ((4, 64, 3, 128, 2048, 1, "out"), SHAPE), ((4, 64, 8, 128, 0, 1, "out"), SHAPE),
    ((4, 64, 8, 96, 2048, 1, "out"), UNSUP), ((4, 24, 8, 128, 2048, 1, "out"), UNSUP),
    ((4, 64, 8, 128, 2048, 9, "out"), UNSUP),
])
def test_attn_splits_rejects(args, code):
    out = ctypes.c_int(0)
    a = list(args)
    a[-1] = None if a[-1] is None else ctypes.byref(out)
    assert lib._lib.dsa_sparse_attn_splits(*a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(out=None), NULL), (dict(idx=None), NULL),
    (dict(rows=-1), SHAPE), (dict(hkv=3), SHAPE), (dict(num_splits=0), SHAPE),
    (dict(k=2, num_splits=4), SHAPE), (dict(scale=float("nan")), SHAPE),
    (dict(num_splits=3), UNSUP), (dict(num_splits=5), UNSUP), (dict(num_splits=16), UNSUP), (dict(d=96), UNSUP),
    (dict(out=A + 2), ALIGN), (dict(out_lse=A + 2), ALIGN), (dict(q=A + 4), ALIGN),
    (dict(rows=0), OK),
])
def test_merged_rejects(kw, code):
    a = dict(q=A, k_cache=A, v_cache=A, block_table=A, row_req=A, idx=A, rows=4, hq=64, hkv=8,
             d=128, k=2048, page_size=64, max_pages=8, scale=0.088, num_splits=4, out=A,
             out_lse=A, dtype=1, stream=None)
    a.update(kw)
    assert lib._lib.dsa_sparse_attn_merged(*a.values()) == code
