"""Test-side helpers: run a step on the GPU and compare it with the oracle.

Expected values come only from ``oracle/``; the inputs it sees are the
generator's tensors, gathered for one row with torch indexing on the device
and copied to the host (the HIP path's outputs are never fed to the oracle).
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import dsa_oracle as O
from sparse_attention_decode_02_amd.step import DsaStep

CANARY = 0x7FBADBAD  # a NaN bit pattern pre-filled into the score buffer

# Output tolerances (max-abs): bf16 inputs 2e-2, fp32 inputs 1e-5; the
# log-sum-exp 1e-3 / 1e-5.
TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}


def run_step(inp, num_splits=None, block_rows=1, canary=True, fused=False, hist=False, **kw):
    step = DsaStep(inp, num_splits=num_splits, block_rows=block_rows, fused=fused, hist=hist, **kw)
    if canary:
        step.scores.view(torch.int32).fill_(CANARY)
    step.run()
    torch.cuda.synchronize()
    return step


def _host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_row(step, r):
    """The oracle's (scores, idx, part_o, part_lse, out, lse) for row r."""
    inp, wl = step.inp, step.wl
    L = int(step.row_len_host[r])
    req = int(step.row_req_host[r])
    dev = inp.q.device
    bt = inp.block_table[req]
    s = torch.arange(L, device=dev)
    kI = _host(inp.kI_cache[bt[s // wl.page].long(), s % wl.page])  # logical keys [L][D_I]
    scores = O.indexer_scores_row(_host(inp.qI[r]), _host(inp.w[r]), kI)
    idx = O.topk_row(scores, L, wl.topk)
    sel = idx[idx >= 0]
    n = len(sel)
    # The selected keys/values as a one-key-per-page cache, slot j = selection j.
    kc = np.zeros((wl.topk, 1, wl.hkv, wl.d))
    vc = np.zeros((wl.topk, 1, wl.hkv, wl.d))
    if n:
        p = torch.from_numpy(sel.astype(np.int64)).to(dev)
        pages = bt[p // wl.page].long()
        kc[:n, 0] = _host(inp.k_cache[pages, p % wl.page])
        vc[:n, 0] = _host(inp.v_cache[pages, p % wl.page])
    local = np.full(wl.topk, -1, np.int64)
    local[:n] = np.arange(n)
    po, pl = O.attention_split_row(_host(inp.q[r]), kc, vc, np.arange(wl.topk), 1, local,
                                   wl.attn_scale, step.num_splits)
    o, lse = O.merge_row(po, pl)
    return scores, idx, po, pl, o, lse


def check_row(step, r):
    """Assert row r of ``step`` matches the oracle; returns the max errors."""
    wl = step.wl
    L = int(step.row_len_host[r])
    tol_o, tol_l = TOL[wl.dtype]
    scores, idx, po, pl, o, lse = oracle_row(step, r)
    got_s = step.scores[r].cpu()
    gs = got_s[:L].numpy()
    assert not np.isnan(gs).any(), f"row {r}: unwritten score positions"
    assert np.array_equal(gs, scores), f"row {r}: scores differ at {np.flatnonzero(gs != scores)[:8]}"
    tail = got_s[L:].view(torch.int32)
    assert bool((tail == CANARY).all()), f"row {r}: a score past the row length was written"
    gi = step.idx[r].cpu().numpy()
    assert np.array_equal(gi, idx), f"row {r}: indices differ at {np.flatnonzero(gi != idx)[:8]}"
    e_po = e_pl = 0.0
    if not step.fused:
        gpo = _host(step.part_o[r])
        gpl = _host(step.part_lse[r])
        e_po = float(np.abs(gpo - po).max()) if po.size else 0.0
        fin = np.isfinite(pl)
        assert np.array_equal(np.isfinite(gpl), fin), f"row {r}: empty splits differ"
        e_pl = float(np.abs(gpl[fin] - pl[fin]).max()) if fin.any() else 0.0
    go = _host(step.out[r])
    gl = _host(step.out_lse[r])
    e_o = float(np.abs(go - o).max())
    finl = np.isfinite(lse)
    assert np.array_equal(np.isfinite(gl), finl)
    e_l = float(np.abs(gl[finl] - lse[finl]).max()) if finl.any() else 0.0
    assert e_po <= tol_o, f"row {r}: partial o error {e_po}"
    assert e_pl <= tol_l, f"row {r}: partial lse error {e_pl}"
    assert e_o <= tol_o, f"row {r}: output error {e_o}"
    assert e_l <= tol_l, f"row {r}: lse error {e_l}"
    return dict(part_o=e_po, part_lse=e_pl, out=e_o, lse=e_l)


def check_properties(step):
    """Size-independent properties of every row's selection, on the device."""
    wl = step.wl
    k = wl.topk
    L = step.row_len.long()[:, None]
    idx = step.idx.long()
    slot = torch.arange(k, device=idx.device)[None, :]
    k_eff = torch.clamp(L, max=k)
    valid = slot < k_eff
    assert bool(((idx >= 0) == valid).all()), "padding is not exactly the slots past min(k, L)"
    assert bool((idx[~valid] == -1).all())
    assert bool(((idx < L) | ~valid).all()), "a selected position is past the row length"
    inc = idx[:, 1:] > idx[:, :-1]
    assert bool((inc | ~valid[:, 1:]).all()), "selections are not strictly ascending"
    # every selected score >= every unselected score (rows with L > k)
    rows = torch.nonzero(step.row_len > k).flatten()
    for r in rows.tolist():
        n = int(step.row_len[r])
        srow = step.scores[r, :n]
        sel = step.idx[r].long()
        mask = torch.ones(n, dtype=torch.bool, device=srow.device)
        mask[sel] = False
        T = srow[sel].min()
        assert float(T) >= float(srow[mask].max()), f"row {r}: not a top-k"
        # ties at the threshold go to the lower positions
        pos = torch.arange(n, device=srow.device)
        tied_out = pos[mask & (srow == T)]
        if tied_out.numel():
            tied_in = sel[srow[sel] == T]
            assert int(tied_in.max()) < int(tied_out.min()), f"row {r}: tie went to a higher position"
