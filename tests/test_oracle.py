"""Pins of the CPU oracle against things other than itself.

Each oracle function is checked against at least one of: values derived by
hand (tests/golden/hand_worked.json), brute-force loops over tiny inputs
written independently here, closed forms, a library routine (torch's
scaled_dot_product_attention in float64 on the CPU), and invariants. The cases
are chosen so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_decode_02_amd import inputs as I


def _f(x):
    return float("-inf") if x == "-inf" else float("inf") if x == "inf" else float(x)


# --------------------------------------------------------------------------
# Hand-worked values
# --------------------------------------------------------------------------


def test_golden_paged_indexer(golden):
    g = golden["paged_indexer"]
    cache = np.asarray(g["kI_cache"], np.float64)
    kI = O.gather_logical(cache, g["block_table"][0], g["row_len"], g["page"])
    s = O.indexer_scores_row(np.asarray(g["qI"]), np.asarray(g["w"]), kI)
    assert s.dtype == np.float32
    assert s.tolist() == g["scores"]
    rows = O.indexer_scores(np.asarray([g["qI"]]), np.asarray([g["w"]]), cache,
                            np.asarray(g["block_table"]), [0], [g["row_len"]], g["page"])
    assert rows[0].tolist() == g["scores"]


def test_golden_topk(golden):
    for c in golden["topk_cases"]:
        sc = np.asarray([_f(x) for x in c["scores"]], np.float32)
        got = O.topk_row(sc, c["len"], c["k"])
        assert got.tolist() == c["idx"], c["why"]


def test_golden_attention(golden):
    g = golden["attention"]
    o, lse = O.attention_row(np.asarray(g["q"]), np.asarray(g["k_cache"], np.float64),
                             np.asarray(g["v_cache"], np.float64), g["block_table"][0],
                             g["page"], np.asarray(g["idx"]), g["scale"])
    np.testing.assert_allclose(o, g["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, g["lse"], rtol=0, atol=1e-14)


def test_golden_merge(golden):
    g = golden["merge"]
    po = np.asarray(g["part_o"])
    pl = np.asarray([[_f(x) for x in r] for r in g["part_lse"]])
    o, lse = O.merge_row(po, pl)
    np.testing.assert_allclose(o, g["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, g["lse"], rtol=0, atol=1e-14)


def test_golden_row_plan(golden):
    g = golden["row_plan"]
    req, ln = O.row_plan(g["prior"], g["new"])
    assert req.tolist() == g["row_req"] and ln.tolist() == g["row_len"]


# --------------------------------------------------------------------------
# Row plan and score blocks
# --------------------------------------------------------------------------


def test_row_plan_properties():
    rng = np.random.default_rng(1)
    prior = rng.integers(0, 50, 9)
    new = rng.integers(1, 6, 9)
    req, ln = O.row_plan(prior, new)
    assert len(req) == new.sum()
    for q in range(9):
        mine = ln[req == q]
        # a request's rows see consecutive causal prefixes ending at its total
        assert mine.tolist() == list(range(prior[q] + 1, prior[q] + new[q] + 1))
    assert np.all(np.diff(req) >= 0)


def test_score_blocks_properties():
    req = np.asarray([0, 0, 0, 0, 0, 1, 2, 2, 2, 3], np.int32)
    b = O.score_blocks(req, 2)
    assert b.tolist() == [[0, 2], [2, 2], [4, 1], [5, 1], [6, 2], [8, 1], [9, 1]]
    b = O.score_blocks(req, 16)
    assert b.tolist() == [[0, 5], [5, 1], [6, 3], [9, 1]]
    assert O.score_blocks(req, 1).tolist() == [[i, 1] for i in range(10)]


# --------------------------------------------------------------------------
# Indexer
# --------------------------------------------------------------------------


def _brute_scores(qI, w, kI_cache, bt_row, L, P):
    """Scalar loops, page by page, written independently of the oracle."""
    H, D = len(qI), len(qI[0])
    out = []
    for s in range(L):
        page, slot = bt_row[s // P], s % P
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for j in range(D):
                dot += float(qI[h][j]) * float(kI_cache[page][slot][j])
            if dot > 0:
                tot += float(w[h]) * dot
        out.append(tot)
    return out


@pytest.mark.parametrize("P", [1, 4, 16])
def test_indexer_brute_force_integers(P):
    rng = np.random.default_rng(7 + P)
    H, D, L = 5, 7, 37
    npages = -(-L // P) + 3
    cache = rng.integers(-4, 5, (npages, P, D)).astype(np.float64)
    bt = rng.permutation(npages)[: -(-L // P)]
    qI = rng.integers(-4, 5, (H, D)).astype(np.float64)
    w = rng.choice([0.5, 1.0, 2.0, -1.0], H)
    got = O.indexer_scores_row(qI, w, O.gather_logical(cache, bt, L, P))
    want = np.asarray(_brute_scores(qI, w, cache, bt, L, P), np.float32)
    assert np.array_equal(got, want)


def test_indexer_brute_force_floats():
    rng = np.random.default_rng(3)
    H, D, L, P = 4, 9, 23, 8
    cache = rng.standard_normal((4, P, D))
    bt = [2, 0, 3]
    qI = rng.standard_normal((H, D))
    w = rng.standard_normal(H)
    got = O.indexer_scores_row(qI, w, O.gather_logical(cache, bt, L, P))
    want = np.asarray(_brute_scores(qI, w, cache, bt, L, P))
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("c", [3.0, -2.0])
def test_indexer_closed_form_unit_query(c):
    """One head, w = 1, qI = c * e_j: score[s] = max(0, c * kI[s][j]), which
    reads key s's j-th element straight through the block table."""
    rng = np.random.default_rng(11)
    P, D, L, j = 4, 6, 14, 4
    cache = rng.integers(-4, 5, (5, P, D)).astype(np.float64)
    bt = [3, 1, 4, 0]
    qI = np.zeros((1, D))
    qI[0, j] = c
    got = O.indexer_scores_row(qI, [1.0], O.gather_logical(cache, bt, L, P))
    for s in range(L):
        assert got[s] == max(0.0, c * cache[bt[s // P], s % P, j])


def test_indexer_relu_before_weight():
    """A negative weight must scale the rectified dot product, not be folded
    inside the ReLU: w = -1 gives -max(0, dot)."""
    kI = np.asarray([[1.0, 0.0], [-1.0, 0.0]])
    s = O.indexer_scores_row([[2.0, 0.0]], [-1.0], kI)
    assert s.tolist() == [-2.0, 0.0]


def test_indexer_head_sum_and_weights_pair_up():
    """Distinct weights per head: swapping two heads' queries without their
    weights changes the result, so the weight index must follow the head."""
    kI = np.asarray([[1.0, 1.0]])
    s1 = O.indexer_scores_row([[1.0, 0.0], [3.0, 0.0]], [1.0, 10.0], kI)
    s2 = O.indexer_scores_row([[3.0, 0.0], [1.0, 0.0]], [1.0, 10.0], kI)
    assert s1.tolist() == [31.0] and s2.tolist() == [13.0]


def test_indexer_page_permutation_invariance():
    wl = I.custom(I.tiny(), prior=(40, 70, 5), new=(1, 1, 1))
    inp = I.generate(wl)
    kc = I.as_f64(inp.kI_cache)
    bt = inp.block_table.numpy()
    qI, w = I.as_f64(inp.qI), I.as_f64(inp.w)
    req, ln = O.row_plan(wl.prior, wl.new)
    a = O.indexer_scores(qI, w, kc, bt, req, ln, wl.page)
    # move every physical page elsewhere and rewrite the table to match
    perm = np.random.default_rng(5).permutation(kc.shape[0])
    kc2 = np.empty_like(kc)
    kc2[perm] = kc
    bt2 = perm[bt]
    b = O.indexer_scores(qI, w, kc2, bt2, req, ln, wl.page)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_indexer_negative_zero_canonical():
    s = O.indexer_scores_row([[1.0]], [-1.0], [[-3.0]])  # -1 * max(0, -3) = -0.0
    assert s[0] == 0.0 and not np.signbit(s[0])


# --------------------------------------------------------------------------
# Top-k
# --------------------------------------------------------------------------


def _brute_topk(scores, L, k):
    keyed = sorted(range(L), key=lambda s: (-(float(scores[s]) + 0.0), s))
    sel = sorted(keyed[: min(k, L)])
    return sel + [-1] * (k - len(sel))


def _threshold_topk(scores, L, k):
    """Second formulation: the k_eff-th largest value T, every position above
    T, then the lowest positions equal to T."""
    v = np.asarray(scores[:L], np.float64) + 0.0
    k_eff = min(k, L)
    if k_eff == 0:
        return [-1] * k
    T = np.sort(v)[::-1][k_eff - 1]
    above = [s for s in range(L) if v[s] > T]
    equal = [s for s in range(L) if v[s] == T][: k_eff - len(above)]
    sel = sorted(above + equal)
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        L = int(rng.integers(0, 60))
        k = int(rng.integers(1, 70))
        sc = rng.integers(-5, 6, max(L, 1) + 3).astype(np.float32) / 2
        if rng.random() < 0.3 and L:
            sc[rng.integers(0, L, 3)] = -np.inf
        if rng.random() < 0.3 and L:
            sc[rng.integers(0, L, 2)] = np.inf
        got = O.topk_row(sc, L, k).tolist()
        assert got == _brute_topk(sc, L, k) == _threshold_topk(sc, L, k)


def test_topk_invariants():
    rng = np.random.default_rng(9)
    L, k = 500, 64
    sc = rng.integers(0, 40, L).astype(np.float32)
    idx = O.topk_row(sc, L, k)
    sel = idx[idx >= 0]
    assert len(sel) == k and np.all(np.diff(sel) > 0) and sel.max() < L
    rest = np.setdiff1d(np.arange(L), sel)
    assert sc[sel].min() >= sc[rest].max()
    T = sc[sel].min()
    # among positions equal to T, the selected ones are the lowest
    eq = np.flatnonzero(sc == T)
    chosen = np.intersect1d(eq, sel)
    assert np.array_equal(chosen, eq[: len(chosen)])
    # top-k is contained in top-(k+1)
    idx2 = O.topk_row(sc, L, k + 1)
    assert set(sel.tolist()) <= set(idx2[idx2 >= 0].tolist())


def test_topk_special_cases():
    L, k = 40, 8
    assert O.topk_row(np.full(L, 3.5, np.float32), L, k).tolist() == list(range(k))
    dec = np.arange(L, 0, -1).astype(np.float32)
    assert O.topk_row(dec, L, k).tolist() == list(range(k))
    inc = np.arange(L).astype(np.float32)
    assert O.topk_row(inc, L, k).tolist() == list(range(L - k, L))
    ninf = np.full(L, -np.inf, np.float32)
    assert O.topk_row(ninf, 5, k).tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert O.topk_row(inc, 0, 3).tolist() == [-1, -1, -1]
    assert O.topk_row(inc, k, k).tolist() == list(range(k))
    assert O.topk_row(inc, k + 1, k).tolist() == list(range(1, k + 1))
    assert O.topk_row(inc, k - 1, k).tolist() == list(range(k - 1)) + [-1]


def test_topk_reads_only_the_length():
    sc = np.asarray([1, 2, 3, 100, 100], np.float32)
    assert O.topk_row(sc, 3, 2).tolist() == [1, 2]


# --------------------------------------------------------------------------
# Attention and merge
# --------------------------------------------------------------------------


def _small_attention_case(seed, L, hq=4, hkv=2, d=8, P=4):
    rng = np.random.default_rng(seed)
    npg = -(-L // P) + 2
    kc = rng.standard_normal((npg, P, hkv, d))
    vc = rng.standard_normal((npg, P, hkv, d))
    bt = rng.permutation(npg)[: -(-L // P)]
    q = rng.standard_normal((hq, d))
    return q, kc, vc, bt, P


@pytest.mark.parametrize("L,hq,hkv", [(1, 4, 2), (13, 4, 2), (30, 8, 1), (17, 6, 3)])
def test_attention_dense_when_topk_covers_length(L, hq, hkv):
    """k >= L selects every key, so the result is plain causal attention over
    [0, L): compare with torch's scaled_dot_product_attention in float64 with
    each KV head repeated for its group of query heads."""
    q, kc, vc, bt, P = _small_attention_case(L, L, hq, hkv)
    k = L + 5
    idx = O.topk_row(np.zeros(L, np.float32), L, k)
    scale = 0.37
    o, lse = O.attention_row(q, kc, vc, bt, P, idx, scale)
    K = O.gather_logical(kc, bt, L, P)  # [L][hkv][d]
    V = O.gather_logical(vc, bt, L, P)
    G = hq // hkv
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    qt = torch.from_numpy(q)[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[0, :, 0, :]
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    z = scale * torch.einsum("hd,hld->hl", torch.from_numpy(q), Kt[0])
    np.testing.assert_allclose(lse, torch.logsumexp(z, -1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("S", [1, 2, 3, 8, 16, 40])
def test_split_merge_equals_unsplit(S):
    q, kc, vc, bt, P = _small_attention_case(4, 33)
    sc = np.random.default_rng(2).standard_normal(33).astype(np.float32)
    idx = O.topk_row(sc, 33, 16)
    o1, l1 = O.attention_row(q, kc, vc, bt, P, idx, 0.5)
    po, pl = O.attention_split_row(q, kc, vc, bt, P, idx, 0.5, S)
    assert po.shape == (4, S, 8) and pl.shape == (4, S)
    o2, l2 = O.merge_row(po, pl)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_split_bounds():
    assert O.split_bounds(10, 3) == [(0, 4), (4, 8), (8, 10)]
    assert O.split_bounds(4, 8) == [(0, 1), (1, 2), (2, 3), (3, 4), (4, 4), (4, 4), (4, 4), (4, 4)]
    assert O.split_bounds(2048, 8)[-1] == (1792, 2048)


def test_attention_single_key_returns_its_value():
    q, kc, vc, bt, P = _small_attention_case(8, 9)
    idx = np.asarray([5, -1, -1], np.int32)
    o, lse = O.attention_row(q * 100, kc, vc, bt, P, idx, 1.0)
    V5 = vc[bt[5 // P], 5 % P]
    G = 2
    for h in range(4):
        assert np.array_equal(o[h], V5[h // G])
    K5 = kc[bt[5 // P], 5 % P]
    np.testing.assert_allclose(lse, [100 * q[h] @ K5[h // G] for h in range(4)], rtol=1e-13)


def test_attention_zero_query_is_mean_of_selected_values():
    q, kc, vc, bt, P = _small_attention_case(9, 20)
    idx = np.asarray([1, 4, 7, 19, -1], np.int32)
    o, lse = O.attention_row(np.zeros_like(q), kc, vc, bt, P, idx, 1.0)
    sel = np.asarray([1, 4, 7, 19])
    V = vc[bt[sel // P], sel % P]  # [4][hkv][d]
    for h in range(4):
        np.testing.assert_allclose(o[h], V[:, h // 2, :].mean(0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(4), rtol=0, atol=1e-14)


def test_attention_slot_permutation_invariance():
    q, kc, vc, bt, P = _small_attention_case(10, 40)
    idx = np.asarray([3, 8, 9, 21, 30, 39, -1, -1], np.int32)
    o1, l1 = O.attention_row(q, kc, vc, bt, P, idx, 0.8)
    o2, l2 = O.attention_row(q, kc, vc, bt, P, idx[[5, 2, 7, 0, 6, 4, 1, 3]], 0.8)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_attention_empty_selection():
    q, kc, vc, bt, P = _small_attention_case(11, 5)
    po, pl = O.attention_split_row(q, kc, vc, bt, P, np.full(6, -1, np.int32), 1.0, 3)
    assert np.all(po == 0) and np.all(pl == -np.inf)
    o, lse = O.merge_row(po, pl)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_attention_gqa_groups_are_contiguous():
    """Heads 0,1 read KV head 0 and heads 2,3 read KV head 1 (h // G): with a
    single selected key, each head's output is its group's value row."""
    kc = np.zeros((1, 2, 2, 3))
    vc = np.zeros((1, 2, 2, 3))
    vc[0, 0, 0] = [1, 2, 3]
    vc[0, 0, 1] = [7, 8, 9]
    o, _ = O.attention_row(np.ones((4, 3)), kc, vc, [0], 2, np.asarray([0]), 1.0)
    assert o.tolist() == [[1, 2, 3], [1, 2, 3], [7, 8, 9], [7, 8, 9]]


def test_merge_single_split_is_identity():
    rng = np.random.default_rng(12)
    po = rng.standard_normal((3, 1, 5))
    pl = rng.standard_normal((3, 1))
    o, lse = O.merge_row(po, pl)
    np.testing.assert_allclose(o, po[:, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, pl[:, 0], rtol=0, atol=1e-15)


def test_merge_two_equal_splits():
    """Two splits with equal lse average their outputs and add ln 2."""
    po = np.asarray([[[1.0, 3.0], [3.0, 5.0]]])
    pl = np.asarray([[0.25, 0.25]])
    o, lse = O.merge_row(po, pl)
    np.testing.assert_allclose(o, [[2.0, 4.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, [0.25 + math.log(2)], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# Whole row on a tiny workload
# --------------------------------------------------------------------------


def test_layer_row_tiny_workload_consistency():
    wl = I.tiny()
    inp = I.generate(wl)
    req, ln = O.row_plan(wl.prior, wl.new)
    assert ln.tolist() == [37, 100]
    args = (req, ln, I.as_f64(inp.qI), I.as_f64(inp.w), I.as_f64(inp.q), I.as_f64(inp.kI_cache),
            I.as_f64(inp.k_cache), I.as_f64(inp.v_cache), inp.block_table.numpy(), wl.page,
            wl.topk, wl.attn_scale)
    for r in range(2):
        s, idx, po, pl, o, lse = O.layer_row(r, *args, num_splits=3)
        assert len(s) == ln[r] and len(idx) == wl.topk
        assert idx.tolist() == _brute_topk(s, ln[r], wl.topk)
        # dyadic integers: scores are multiples of 0.5
        assert np.all(np.asarray(s) * 2 == np.round(np.asarray(s) * 2))
        o1, l1 = O.attention_row(I.as_f64(inp.q)[r], I.as_f64(inp.k_cache), I.as_f64(inp.v_cache),
                                 inp.block_table.numpy()[req[r]], wl.page, idx, wl.attn_scale)
        np.testing.assert_allclose(o, o1, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Score histogram (the selection's exact threshold)
# --------------------------------------------------------------------------


def test_golden_order_key_bins(golden):
    g = golden["order_key_bins"]["cases"]
    sc = np.asarray([_f(c["score"]) for c in g], np.float32)
    keys = O.order_keys(sc)
    assert keys.tolist() == [c["key"] for c in g]
    h = O.score_histogram_row(sc, len(sc))
    want = np.zeros(4096, np.int64)
    for c in g:
        want[c["bin"]] += 1
    assert np.array_equal(h, want)


def test_order_keys_brute_force():
    """Each key from the bit pattern, one value at a time (struct), and the
    key order equals the value order over all kinds of float32."""
    import struct
    rng = np.random.default_rng(4)
    vals = np.concatenate([
        rng.standard_normal(200) * 10.0 ** rng.integers(-40, 38, 200),
        [0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38, -3.4e38, 1.0, -1.0],
        np.round(rng.normal(2240, 400, 100) * 2) / 2]).astype(np.float32)
    for v in vals:
        b = struct.unpack("<I", struct.pack("<f", float(v)))[0]
        if b == 0x80000000:
            b = 0
        want = (b ^ 0xFFFFFFFF) if b >> 31 else (b | 0x80000000)
        assert int(O.order_keys(np.asarray([v], np.float32))[0]) == want
    order = np.argsort(vals.astype(np.float64), kind="stable")
    k = O.order_keys(vals)[order]
    assert np.all(np.diff(k) >= 0)
    eq = np.diff(vals.astype(np.float64)[order]) == 0
    assert np.all((np.diff(k) == 0) == eq)


@pytest.mark.parametrize("seed", range(6))
def test_score_histogram_threshold_bin(seed):
    """The histogram counts exactly the row's first L scores, and the bin
    where the count from the top reaches k holds the k-th largest score -- the
    smallest score the top-k selects."""
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 5000))
    width = L + int(rng.integers(0, 100))
    sc = (rng.integers(-50, 400, width) / 4).astype(np.float32)
    sc[L:] = np.nan
    h = O.score_histogram_row(sc, L)
    assert int(h.sum()) == L
    brute = np.zeros(4096, np.int64)
    for v in sc[:L]:
        brute[int(O.order_keys(np.asarray([v], np.float32))[0]) >> 20] += 1
    assert np.array_equal(h, brute)
    for k in (1, 7, min(L, 100), L):
        top = np.cumsum(h[::-1])
        b = 4095 - int(np.argmax(top >= k))
        sel = O.topk_row(sc, L, k)
        kth = sc[sel[sel >= 0]].min()
        assert int(O.order_keys(np.asarray([kth], np.float32))[0]) >> 20 == b
        assert int(top[4095 - b]) - int(h[b]) < k <= int(top[4095 - b])
