"""CPU model of the top-k kernel's selection arithmetic, against the oracle.

The selection kernel finds a threshold prefix by radix passes and then writes
the winners with an ordered compaction: every thread counts its keys above the
prefix and equal to it, a block-wide exclusive scan of those counts gives each
thread its first output slots, and each thread walks its own keys in position
order. This module re-enacts that arithmetic with NumPy for a workgroup of
``threads`` threads holding ``vpt`` consecutive positions each per chunk (the
shapes the library launches), and compares the slots it produces with the
oracle's top-k (stable sort, ties to the lower position).

The count scan is modelled at a given field width. The kernel packs the two
counts as 16-bit fields of one word when a chunk holds fewer than 65536 keys
(no count or prefix sum can reach 65536 there) and scans them at full 32-bit
width for the 65536-key chunk, where the packing would lose a carry when all
keys tie with the threshold. The model shows all three: full width and the
kernel's rule match the oracle on every row at every launched shape, and the
16-bit packing fails on the fully tied 65536-key chunks.
"""

import numpy as np
import pytest

from oracle import dsa_oracle as O

KMASK = (1 << 32) - 1


def order_keys(scores):
    """Order-preserving 32-bit keys (int64 holding uint32), -0.0 as +0.0."""
    u = np.asarray(scores, np.float32).view(np.uint32).astype(np.int64)
    u = np.where(u == 0x80000000, 0, u)
    return np.where(u & 0x80000000, (~u) & KMASK, u | 0x80000000)


def radix_threshold(keys, k):
    """The kernel's radix passes: (shift, prefix, need) of the threshold."""
    mx, mn = int(keys.max()), int(keys.min())
    if mx == mn:
        return 0, mx, k
    shift = (mx ^ mn).bit_length()
    prefix = mx >> shift if shift < 32 else 0
    # bits below the lowest one where two keys differ are shared by all keys
    varying = int(np.bitwise_or.reduce(keys)) ^ int(np.bitwise_and.reduce(keys))
    low = (varying & -varying).bit_length() - 1
    need = k
    first = True
    while shift > low:
        nb = min(12, shift - low)
        ns = shift - nb
        cand = keys if first else keys[(keys >> shift) == prefix]
        hist = np.bincount((cand >> ns) & ((1 << nb) - 1), minlength=1 << nb)
        above = 0
        for digit in range((1 << nb) - 1, -1, -1):
            if above + hist[digit] >= need:
                break
            above += int(hist[digit])
        prefix = (prefix << nb) | digit
        shift = ns
        need -= above
        first = False
        if int(hist[digit]) == need:
            break
    return shift, prefix, need


def emit(keys, k, threads, vpt, field_bits=None):
    """The ordered compaction; field_bits=16 packs the two counts into one
    32-bit word as (above << 16) | tied, None scans them at full width."""
    L = len(keys)
    shift, prefix, need = radix_threshold(keys, k)
    out = np.full(k, -7, np.int64)
    chunk = threads * vpt
    gt_run = eq_run = 0
    for c0 in range(0, L, chunk):
        pos = c0 + np.arange(chunk).reshape(threads, vpt)
        valid = pos < L
        kk = np.where(valid, keys[np.minimum(pos, L - 1)], 0)
        hb = kk >> shift
        gt = (hb > prefix) & valid
        eq = (hb == prefix) & valid
        cg, ce = gt.sum(1).astype(np.int64), eq.sum(1).astype(np.int64)
        if field_bits is None:
            xg, xe = np.cumsum(cg) - cg, np.cumsum(ce) - ce
            tg, te = int(cg.sum()), int(ce.sum())
        else:
            packed = ((cg << field_bits) | ce) & KMASK
            excl = (np.cumsum(packed) - packed) & KMASK
            total = int(packed.sum()) & KMASK
            low = (1 << field_bits) - 1
            xg, xe = excl >> field_bits, excl & low
            tg, te = total >> field_bits, total & low
        g = gt_run + xg[:, None] + (np.cumsum(gt, 1) - gt)
        e = eq_run + xe[:, None] + (np.cumsum(eq, 1) - eq)
        slot_gt = g + np.minimum(e, need)
        w = gt & (slot_gt < k)
        out[slot_gt[w]] = pos[w]
        w = eq & (e < need) & (g + e < k)
        out[(g + e)[w]] = pos[w]
        gt_run += tg
        eq_run += te
    return out


def kernel_field_bits(threads, vpt):
    """The kernel's choice: one packed word below 65536 keys per chunk."""
    return 16 if threads * vpt < 65536 else None


def _rows():
    rng = np.random.default_rng(3)
    tail = np.concatenate([np.zeros(65536, np.float32), (rng.random(100) + 1).astype(np.float32)])
    return [
        ("70000 equal", np.full(70000, 7.5, np.float32)),
        ("70000 zeros", np.zeros(70000, np.float32)),
        ("65536 zeros then positives", tail),
        ("65536 equal", np.full(65536, -2.0, np.float32)),
        ("normal 70000", rng.standard_normal(70000).astype(np.float32)),
        ("ties 70000", (rng.integers(0, 300, 70000) / 2).astype(np.float32)),
    ]


# (threads, keys per thread): the whole-row, segment and gather shapes launched
SHAPES = [(1024, 64), (1024, 32), (512, 64), (512, 16)]


@pytest.mark.parametrize("threads,vpt", SHAPES)
@pytest.mark.parametrize("k", [16, 2048])
def test_full_width_scan_matches_oracle(threads, vpt, k):
    for name, sc in _rows():
        want = O.topk_row(sc, len(sc), k)
        got = emit(order_keys(sc), k, threads, vpt)
        assert np.array_equal(got, want), (name, np.flatnonzero(got != want)[:5])


@pytest.mark.parametrize("threads,vpt", SHAPES)
@pytest.mark.parametrize("k", [16, 2048])
def test_kernel_scan_width_matches_oracle(threads, vpt, k):
    """What the kernel does at each shape: packed counts for the 32768-key
    and smaller chunks, full width for the 65536-key chunk."""
    fb = kernel_field_bits(threads, vpt)
    assert (fb is None) == (threads * vpt == 65536)
    for name, sc in _rows():
        want = O.topk_row(sc, len(sc), k)
        got = emit(order_keys(sc), k, threads, vpt, field_bits=fb)
        assert np.array_equal(got, want), (name, np.flatnonzero(got != want)[:5])


@pytest.mark.parametrize("k", [16, 2048])
def test_packed_16bit_counts_fail_on_tied_full_chunk(k):
    """The 16-bit packing is wrong exactly where a 65536-key chunk fully ties
    (and right where no chunk does): the rows above reach that case."""
    bad = []
    for name, sc in _rows():
        want = O.topk_row(sc, len(sc), k)
        got = emit(order_keys(sc), k, 1024, 64, field_bits=16)
        if not np.array_equal(got, want):
            bad.append(name)
    assert set(bad) == {"70000 equal", "70000 zeros", "65536 zeros then positives"} - (
        {"65536 zeros then positives"} if k <= 100 else set())


def test_radix_passes_skip_shared_low_bits():
    """Dyadic scores with short significands share their low key bits: the
    passes stop above them and still find the k-th key."""
    rng = np.random.default_rng(5)
    sc = (np.round(rng.normal(2240, 400, 32768) * 2) / 2).astype(np.float32)
    keys = order_keys(sc)
    shift, prefix, need = radix_threshold(keys, 2048)
    assert shift >= 11
    kth = np.sort(keys)[::-1][2047]
    assert (kth >> shift) == prefix
    assert np.array_equal(emit(keys, 2048, 1024, 32), O.topk_row(sc, len(sc), 2048))


def test_radix_threshold_is_the_kth_key():
    rng = np.random.default_rng(9)
    for _ in range(20):
        sc = rng.integers(-50, 50, int(rng.integers(20, 3000))).astype(np.float32) / 4
        k = int(rng.integers(1, len(sc)))
        keys = order_keys(sc)
        shift, prefix, need = radix_threshold(keys, k)
        kth = np.sort(keys)[::-1][k - 1]
        assert (kth >> shift) == prefix
        assert int(((keys >> shift) > prefix).sum()) == k - need
