"""The allocation-free two-stage top-k (dsa_topk_chunked_noalloc) against
dsa_topk_chunked with a caller workspace, through the C ABI: two calls in a
row on one device, the second with a smaller input, each bit for bit equal to
the workspace call and, on sampled rows, to the oracle."""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu


def _batch(rows, width, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, width + 1, rows).astype(np.int32)
    lens[0] = width
    scores = np.full((rows, width), np.nan, np.float32)
    for i in range(rows):
        scores[i, : lens[i]] = (rng.integers(0, 400, lens[i]) / 4).astype(np.float32)
    scores[1, : lens[1]] = 0.0  # a fully tied row
    return scores, lens


@pytest.mark.parametrize("calls", [[(24, 70016, 2048, 8192, 1), (5, 20000, 16, 4096, 2)]],
                         ids=["large-then-small"])
def test_noalloc_matches_workspace_call(calls):
    assert torch.cuda.is_available(), "GPU test"
    from sparse_attention_decode_02_amd import lib
    for rows, width, k, chunk, seed in calls:
        print(f"noalloc top-k: rows {rows} width {width} k {k} chunk {chunk}", flush=True)
        assert lib.topk_chunked_slots(rows, width, k, chunk) <= lib.TOPK_NOALLOC_MAX_SLOTS
        scores, lens = _batch(rows, width, seed)
        s_d = torch.from_numpy(scores).cuda()
        l_d = torch.from_numpy(lens).cuda()
        cand = torch.full((lib.topk_chunked_slots(rows, width, k, chunk),), -9, dtype=torch.int32,
                          device="cuda")
        ref = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        lib.topk_chunked(s_d, l_d, k, chunk, cand, ref)
        got = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        lib.topk_chunked_noalloc(s_d, l_d, k, chunk, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        g = got.cpu().numpy()
        for r in (0, 1, rows - 1):
            want = O.topk_row(scores[r], int(lens[r]), k)
            assert np.array_equal(g[r], want), r


def test_noalloc_rejects_oversized_and_bad_arguments():
    from sparse_attention_decode_02_amd import lib
    s = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    l_d = torch.full((2,), 64, dtype=torch.int32, device="cuda")
    idx = torch.zeros((2, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(lib.DsaError) as e:
        lib.topk_chunked_noalloc(s, l_d, 16, 8, idx)  # chunk < k
    assert e.value.status == -2
    big = torch.zeros((2048, 4096), dtype=torch.float32, device="cuda")
    lb = torch.full((2048,), 4096, dtype=torch.int32, device="cuda")
    ib = torch.zeros((2048, 2048), dtype=torch.int32, device="cuda")
    with pytest.raises(lib.DsaError) as e:
        lib.topk_chunked_noalloc(big, lb, 2048, 2048, ib)  # 2 * 2048 * 2 * 2048 slots > max
    assert e.value.status == -5
