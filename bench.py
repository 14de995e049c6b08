"""Benchmark of one paged DSA layer step on one MI355X.

A step is the whole hot path over one batch: indexer scores -> top-k ->
GQA sparse attention (split over the k slots) -> log-sum-exp merge: three
library calls on one stream when the attention splits fit one workgroup
(attention and merge fused in dsa_sparse_attn_merged), four otherwise or with
--unfused. The default workload is batch 64 decode at
context 32768, page 64, 64 query / 8 KV heads of dim 128, indexer 64 x 128,
top-k 2048, bf16, synthetic inputs drawn on the device (randomly permuted
page tables). Inputs are resident in HBM before the timed region; W warm-up
steps run untimed, then K steps are timed between two synchronizations.

Prints one JSON line:
  value          layer latency in microseconds (lower is better)
  hbm_gbps       algorithmic bytes of the layer / latency
  roofline       the dominant kernel's algorithmic bytes per launch / its
                 average duration (HIP events on the launch stream), against
                 8 TB/s
  cpu_baseline   the CPU oracle timed on a bounded sample of rows of the same
                 workload (paged gathers included), extrapolated to the whole
                 layer, on every core this process may use and on one core
  configs        latency, GB/s and fraction of 8 TB/s of the other workloads
                 (tiny, decode, ragged, mixed), measured in the same run
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA layer latency (us) + HBM GB/s, B=64 ctx 32k top-k 2048, 1 GPU"
PROFILE = os.path.join(ROOT, "profiles", "dsa_kernels_decode_b64_ctx32k.json")
STAGE_SOURCE = {"indexer": "indexer.hip", "topk": "topk.hip", "attention": "sparse_attn.hip",
                "merge": "merge.hip"}
HBM_PEAK_GBPS = 8000.0
PAGES_LAYER_US = 160.0  # one decode layer, batch 64, 32K context, top-k 2048, on GB300 (context)


def algorithmic_bytes(wl, row_len):
    """Bytes the method itself must move, per kernel, summed over rows:
    indexer: keys L*D_I*e, qI H_I*D_I*e, w 4*H_I, score write 4*L, block table 4*ceil(L/P)
    top-k:   score read 4*L, index write 4*k
    attention: K and V of the k_eff selected keys k_eff*Hkv*d*e*2, q Hq*d*e,
               index read 4*k, block table 4*ceil(L/P)
    merge:   output write Hq*d*e
    (split partials are overhead, not counted)."""
    e = 2 if wl.dtype == "bf16" else 4
    b = {"indexer": 0, "topk": 0, "attention": 0, "merge": 0}
    for L in (int(x) for x in row_len):
        pages = -(-L // wl.page)
        k_eff = min(wl.topk, L)
        b["indexer"] += L * wl.di * e + wl.hi * wl.di * e + 4 * wl.hi + 4 * L + 4 * pages
        b["topk"] += 4 * L + 4 * wl.topk
        b["attention"] += k_eff * wl.hkv * wl.d * e * 2 + wl.hq * wl.d * e + 4 * wl.topk + 4 * pages
        b["merge"] += wl.hq * wl.d * e
    return b


def profiled_traffic(stage, workload_name):
    """HBM bytes per launch of `stage` from the committed rocprofv3 counter
    summary, or None when there is none for this workload or the kernel's
    source changed since the counters were taken."""
    import hashlib
    if workload_name != "decode_b64_ctx32k_bf16" or not os.path.exists(PROFILE):
        return None
    with open(PROFILE) as f:
        prof = json.load(f)
    src = os.path.join(ROOT, "sparse_attention_decode_02_amd", "csrc", STAGE_SOURCE[stage])
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    for k in prof["kernels"].values():
        if k["stage"] == stage and k["source_sha256"] == sha:
            return int(round(k["hbm_bytes_per_launch"]))
    return None


def attention_label(step):
    """Which attention kernels the step runs: bf16 rows with d 128 and eight
    query heads per KV group go to the matrix-core kernel, other shapes to
    the vector kernel; prefill score blocks may go to group attention."""
    wl = step.wl
    kern = ("matrix-core kernel" if wl.dtype == "bf16" and wl.d == 128 and wl.hq == 8 * wl.hkv
            else "vector kernel")
    merge = "fused merge" if step.fused else "separate merge"
    if step.groups is not None:
        return (f"prefill groups over the union of their selections (matrix cores), "
                f"{step.rows - step.group_rows} rows on the {kern}, {merge}")
    return f"{kern}, {merge}"


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_steps(step, steps, warmup, torch, graph=None, trace=None):
    """Mean step time (ms) of ``steps`` steps after ``warmup``, one event
    before and one after. With a ``trace`` list, events between the steps
    (recorded on the same stream, so they add no wait) give each step's time
    in microseconds too."""
    run = graph.replay if graph is not None else step.run
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [_events(torch)[0] for _ in range(steps + 1)] if trace is not None else None
    a, b = _events(torch)
    a.record()
    for i in range(steps):
        if evs:
            evs[i].record()
        run()
    if evs:
        evs[steps].record()
    b.record()
    torch.cuda.synchronize()
    if evs:
        trace.extend(round(1000.0 * evs[i].elapsed_time(evs[i + 1]), 1) for i in range(steps))
    return a.elapsed_time(b) / steps  # ms


def time_per_step(step, steps, torch, scrub=None):
    """Each step's time in microseconds (HIP events around it alone); with
    ``scrub`` (a device tensor larger than L2 and the Infinity Cache) it is
    read once before every step, outside the events, so the step starts
    with none of its data cached (and no dirty lines to write back)."""
    from sparse_attention_decode_02_amd import lib
    evs = [_events(torch) for _ in range(steps)]
    sink = torch.empty(4096, dtype=torch.float32, device="cuda")
    for i in range(steps):
        if scrub is not None:
            lib.read_probe(scrub, sink)
        evs[i][0].record()
        step.run()
        evs[i][1].record()
    torch.cuda.synchronize()
    return sorted(1000.0 * a.elapsed_time(b) for a, b in evs)


def _pct(v, q):
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def read_floor_gbps(torch, mib=1024, reps=200):
    """A plain streaming read of ``mib`` MiB (dsa_read_probe): the practical
    read bandwidth the layer's GB/s is compared with."""
    from sparse_attention_decode_02_amd import lib
    x = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    sink = torch.empty(4096, dtype=torch.float32, device="cuda")
    for _ in range(3):
        lib.read_probe(x, sink)
    torch.cuda.synchronize()
    a, b = _events(torch)
    a.record()
    for _ in range(reps):
        lib.read_probe(x, sink)
    b.record()
    torch.cuda.synchronize()
    gbps = (mib << 20) * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del x
    return gbps


def time_kernels(step, steps, torch):
    """Average duration of each stage's kernel, HIP events on the launch stream."""
    stages = [("indexer", step.indexer), ("topk", step.topk), ("attention", step.attention)]
    if not step.fused:
        stages.append(("merge", step.merge))
    evs = {n: [_events(torch) for _ in range(steps)] for n, _ in stages}
    for i in range(steps):
        for n, fn in stages:
            evs[n][i][0].record()
            fn()
            evs[n][i][1].record()
    torch.cuda.synchronize()
    return {n: 1000.0 * sum(a.elapsed_time(b) for a, b in evs[n]) / steps for n, _ in stages}


class _Bf16Host:
    """A bf16 tensor held on the host as its raw 16-bit words. Indexing it
    returns the float64 values (exact), so the oracle's own paged gathers
    read the caches through the block table as they would a float array."""

    def __init__(self, words):
        self.words = words
        self.shape = words.shape

    def __getitem__(self, key):
        import numpy as np
        u = np.asarray(self.words[key]).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)


def _host_tensor(t, torch):
    """Host copy of a device tensor for the oracle: bf16 as _Bf16Host, other
    dtypes as NumPy arrays."""
    if t.dtype == torch.bfloat16:
        return _Bf16Host(t.view(torch.int16).cpu().numpy().view("uint16"))
    return t.cpu().numpy()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pass(step, host, rows_order, budget_s):
    """Runs the oracle over rows in the given order until the budget is
    spent. Timed per row: the paged gathers of the indexer keys and of the
    selected K/V (through the block table), the indexer, the top-k, the split
    attention and the merge. Returns (seconds, rows done, their lengths)."""
    from oracle import dsa_oracle as O
    wl = step.wl
    kI_c, k_c, v_c, bt, qI, w, q = host
    spent, done, lens = 0.0, [], []
    for r in rows_order:
        L = int(step.row_len_host[r])
        req = int(step.row_req_host[r])
        t0 = time.perf_counter()
        kI = O.gather_logical(kI_c, bt[req], L, wl.page)
        sc = O.indexer_scores_row(qI[r], w[r], kI)
        idx = O.topk_row(sc, L, wl.topk)
        po, pl = O.attention_split_row(q[r], k_c, v_c, bt[req], wl.page, idx, wl.attn_scale,
                                       step.num_splits)
        O.merge_row(po, pl)
        spent += time.perf_counter() - t0
        done.append(r)
        lens.append(L)
        if spent >= budget_s:
            break
    return spent, done, lens


def cpu_baseline(step, budget_s, torch):
    """The oracle, as it stands, on a bounded sample of rows of this workload:
    once with the BLAS on every host core this process may use (capped by
    OMP_NUM_THREADS when set) and once on one core. Each run takes about
    ``budget_s`` seconds and is scaled to the whole layer by the sampled rows'
    share of its keys."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    inp = step.inp
    affinity = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(affinity, int(env)) if env.isdigit() and int(env) > 0 else affinity
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    host = (_host_tensor(inp.kI_cache, torch), _host_tensor(inp.k_cache, torch),
            _host_tensor(inp.v_cache, torch), inp.block_table.cpu().numpy(),
            f64(inp.qI), f64(inp.w), f64(inp.q))
    rng = np.random.default_rng(0)
    order = np.concatenate([rng.permutation(step.rows) for _ in range(64)]).tolist()
    total_len = float(sum(int(x) for x in step.row_len_host)) or 1.0
    out = {}
    for n in (threads, 1):
        with threadpool_limits(limits=n):
            spent, done, lens = _oracle_pass(step, host, order, budget_s)
        share = sum(lens) / total_len
        out[n] = (spent / share if share > 0 else spent, spent, len(done), len(set(done)), share)
    est, spent, n_done, n_distinct, share = out[threads]
    est1, spent1, n1, _, share1 = out[1]
    return {
        "value": round(est * 1e6, 1),
        "unit": "us",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n_done} row evaluations ({n_distinct} distinct of {step.rows} rows), "
                   f"{spent:.1f} s on {threads} threads, scaled to the layer by their share of "
                   f"its keys ({share:.3f}); timed per row: paged gathers through the block "
                   f"table, indexer, top-k, split attention, merge (float64 NumPy)"),
        "one_core": {"value": round(est1 * 1e6, 1), "unit": "us",
                     "sample": f"{n1} row evaluations, {spent1:.1f} s, share {share1:.3f}"},
        "cpu_model": _cpu_model(),
        "host_cores_available": affinity,
    }


def measure_configs(names, steps, warmup, torch):
    """Latency, algorithmic GB/s and fraction of 8 TB/s for other workloads,
    each generated on the device and timed like the headline (the bench's
    default step configuration), then freed."""
    from sparse_attention_decode_02_amd import inputs as I
    from sparse_attention_decode_02_amd.step import DsaStep
    out = {}
    for spec in names:
        name, _, opt = spec.partition("+")
        # the step's automatic top-k, or the histogram selection forced on / off
        hist = True if opt == "hist" else False if opt == "onepass" else None
        # the step's automatic choice, or group attention forced on / off
        group = True if opt == "group" else False if opt == "split" else None
        wl = I.WORKLOADS[name]()
        print(f"[bench] config {wl.name}{' (histogram top-k)' if hist else ' (one-pass top-k)' if hist is False else ''}"
              f"{' (group attention)' if group else ' (split attention only)' if group is False else ''}",
              file=sys.stderr, flush=True)
        inp = I.generate(wl, "cuda")
        step = DsaStep(inp, block_rows=8, fused=None, topk_chunk=0 if hist is not None else None, hist=hist,
                       group_attn=group)
        torch.cuda.synchronize()
        ms = time_steps(step, steps, warmup, torch)
        kern = time_kernels(step, max(5, steps // 4), torch)
        ab = algorithmic_bytes(wl, step.row_len_host)
        total = sum(ab.values())
        us = ms * 1000.0
        gbps = total / (us * 1e-6) / 1e9
        rec = {"workload": wl.name, "rows": step.rows, "latency_us": round(us, 2),
               "algorithmic_bytes": total, "gbps": round(gbps, 1),
               "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
               "kernels_us": {n: round(v, 2) for n, v in kern.items()},
               "attention_splits": step.num_splits,
               "attention": attention_label(step),
               "topk_mode": ("from the indexer's score histogram" if step.use_hist else
                             f"two-stage, {step.topk_chunk}-position segments"
                             if step.topk_chunk else "one pass")}
        if len(set(step.row_req_host.tolist())) < step.rows:
            # Rows of one request share its keys: the bytes HBM must deliver
            # at least (each request's indexer keys and distinct selected K/V
            # once) are far fewer than the per-row bytes the method issues,
            # most of which the caches serve. GB/s and the fraction of the
            # peak are taken on the compulsory bytes.
            comp = compulsory_bytes(step, wl, torch)
            cg = comp / (us * 1e-6) / 1e9
            rec.update({"algorithmic_bytes": comp, "gbps": round(cg, 1),
                        "frac_of_hbm_peak": round(cg / HBM_PEAK_GBPS, 4),
                        "method_issued_bytes": total, "method_issued_gbps": round(gbps, 1),
                        "bytes_note": ("algorithmic_bytes: each request's indexer keys and "
                                       "distinct selected K/V rows once, every row's scores, "
                                       "queries, indices and outputs; method_issued_bytes: "
                                       "every row's own key reads and gathers")})
        out[spec] = rec
        del step, inp
        torch.cuda.empty_cache()
    return out


def compulsory_bytes(step, wl, torch):
    """Bytes a step must move at least when rows share a request: each
    request's indexer keys once (its longest row), every row's score write
    and read, qI, w, q, out and indices, and each request's distinct selected
    K/V rows once."""
    e = 2 if wl.dtype == "bf16" else 4
    req = step.row_req_host
    lens = step.row_len_host
    b = 0
    longest = {}
    for q, L in zip(req.tolist(), lens.tolist()):
        longest[q] = max(longest.get(q, 0), L)
    for L in longest.values():
        b += L * wl.di * e + 4 * -(-L // wl.page)
    b += int(sum(8 * int(L) for L in lens))  # scores written, read
    b += step.rows * (wl.hi * wl.di * e + 4 * wl.hi + 2 * wl.hq * wl.d * e + 8 * wl.topk)
    idx = step.idx
    rq = step.row_req.long()
    for q in longest:
        sel = idx[rq == q]
        n = int(torch.unique(sel[sel >= 0]).numel())
        b += n * wl.hkv * wl.d * e * 2
    return int(b)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (the first ~20 ms of work run at lower clocks)")
    ap.add_argument("--workload", default="headline",
                    help="headline (default), decode, tiny, ragged, mixed, long or prefill_1m")
    ap.add_argument("--splits", type=int, default=0, help="attention splits (0 = default)")
    ap.add_argument("--block-rows", type=int, default=8,
                    help="most rows of one request per indexer score block (1 = none)")
    ap.add_argument("--unfused", action="store_true",
                    help="always run attention and merge as two launches (dsa_sparse_attn + dsa_merge)")
    ap.add_argument("--topk-chunk", type=int, default=-1,
                    help="top-k segment length for the two-stage selection (0 = one pass, "
                         "-1 = the library's suggestion)")
    ap.add_argument("--score-buffer-mib", type=int, default=0,
                    help="score and select in row windows through a buffer of this many MiB "
                         "(0 = every row at once)")
    ap.add_argument("--hist", type=int, default=-1,
                    help="1: the indexer counts each row's scores and the top-k starts from the "
                         "counts (dsa_indexer_scores_hist + dsa_topk_hist); 0: the one-pass or "
                         "two-stage top-k; -1 (default): the step's automatic choice")
    ap.add_argument("--group-attn", type=int, default=-1,
                    help="1: attention of multi-row score blocks over the union of their "
                         "selections on the matrix cores (dsa_group_attn); 0: every row on the "
                         "split attention kernel; -1 (default): the step's automatic choice")
    ap.add_argument("--graph", action="store_true",
                    help="record the step into a HIP graph once and time its replays")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle time budget for cpu_baseline, per core setting (0 = skip)")
    ap.add_argument("--configs",
                    default="tiny,decode,ragged,mixed,ragged+onepass,mixed+split,long,long+hist",
                    help="other workloads measured in the same run (comma list, '' = none; "
                         "name+hist / name+onepass: with the histogram top-k forced on / off; "
                         "name+group / name+split: group attention forced on / off)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the step, run a plain device copy of this many MiB "
                         "(calibrates HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(requests shard across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": args.warmup + args.steps}))
        return 0

    from sparse_attention_decode_02_amd import inputs as I
    from sparse_attention_decode_02_amd.step import DsaStep

    wl = I.WORKLOADS[args.workload]()
    print(f"[bench] generating {wl.name} on the device", file=sys.stderr, flush=True)
    inp = I.generate(wl, "cuda")
    block_rows = args.block_rows
    opts = dict(num_splits=args.splits or None, block_rows=block_rows,
                fused=False if args.unfused else None,
                topk_chunk=None if args.topk_chunk < 0 else args.topk_chunk,
                score_buffer_bytes=(args.score_buffer_mib << 20) if args.score_buffer_mib else None,
                hist=None if args.hist < 0 else bool(args.hist),
                group_attn=None if args.group_attn < 0 else bool(args.group_attn))
    step = DsaStep(inp, **opts)
    torch.cuda.synchronize()
    print(f"[bench] rows {step.rows} width {step.width} splits {step.num_splits}",
          file=sys.stderr, flush=True)

    graph = step.capture() if args.graph else None
    # The read floor is measured first, over ~33 ms of streaming reads: this
    # also brings the GPU toward its working clocks, which it otherwise
    # reaches only ~15 ms into a run (steps timed right after a short warm-up
    # measure up to ~5% slower than the same steps later in the run).
    floor = read_floor_gbps(torch, reps=200)
    # The per-kernel and single-step measurements come next; they also run
    # the step's kernels long enough for the clocks to settle (after the
    # floor alone the first few dozen steps still run up to ~5% slower), so
    # the timed steps measure the sustained rate.
    warm = time_per_step(step, args.steps, torch)
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB > L2 + MALL
    cold = time_per_step(step, args.steps, torch, scrub)
    del scrub
    kern = time_kernels(step, args.steps, torch)
    # The timed steps carry no events between them: each timing event is a
    # barrier with a cache write-back on the stream, ~3 us per step at the
    # headline. Each step's own time comes from a second pass afterwards.
    ms = time_steps(step, args.steps, args.warmup, torch, graph)
    trace = []
    time_steps(step, args.steps, 0, torch, graph, trace)
    layer_us = ms * 1000.0
    ab = algorithmic_bytes(wl, step.row_len_host)
    total_bytes = sum(ab.values())
    if step.fused:  # the merged kernel also writes the output
        ab["attention"] += ab.pop("merge")
    gbps = total_bytes / (layer_us * 1e-6) / 1e9
    dominant = max(("indexer", "attention"), key=lambda n: kern[n])
    dom_gbps = ab[dominant] / (kern[dominant] * 1e-6) / 1e9
    print(f"[bench] layer {layer_us:.1f} us, {gbps:.0f} GB/s; kernels (us) "
          + ", ".join(f"{n} {v:.1f}" for n, v in kern.items())
          + f"; per step warm {_pct(warm, 0.5):.1f} cold {_pct(cold, 0.5):.1f} us; "
          f"read floor {floor:.0f} GB/s", file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": round(layer_us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(layer_us / PAGES_LAYER_US, 4) if args.workload == "headline" else None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch_rows": step.rows,
            "context": int(max(step.row_len_host)),
            "topk": wl.topk,
            "page": wl.page,
            "q_heads": wl.hq,
            "kv_heads": wl.hkv,
            "head_dim": wl.d,
            "indexer": f"{wl.hi}x{wl.di}",
            "attention_splits": step.num_splits,
            "indexer_block_rows": block_rows,
            "attention_merge": "fused" if step.fused else "separate",
            "launch": "graph replay" if args.graph else "stream",
            "topk_mode": ("from the indexer's score histogram" if step.use_hist else
                          f"two-stage, {step.topk_chunk}-position segments" if step.topk_chunk
                          else "one pass"),
            "score_rows_per_window": step.window_rows,
            "attention": attention_label(step),
        },
        "hbm_gbps": round(gbps, 1),
        "layer_frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "per_step_us": {
            "warm": {"median": round(_pct(warm, 0.5), 2), "p10": round(_pct(warm, 0.1), 2),
                     "p90": round(_pct(warm, 0.9), 2)},
            "cold": {"median": round(_pct(cold, 0.5), 2), "p10": round(_pct(cold, 0.1), 2),
                     "p90": round(_pct(cold, 0.9), 2),
                     "note": "a 1 GiB buffer is read before each step, outside its events"},
        },
        "timed_steps_us": trace,  # a second pass of as many steps, events between them
        "read_floor_gbps": round(floor, 1),
        "layer_frac_of_read_floor": round(gbps / floor, 4),
        "algorithmic_bytes": total_bytes,
        "kernels_us": {n: round(v, 2) for n, v in kern.items()},
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": round(dom_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": profiled_traffic(dominant, wl.name),
            "algorithmic_bytes_per_launch": ab[dominant],
        },
    }
    if args.cpu_seconds > 0:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds, torch)
    this = args.workload + ("+hist" if args.hist > 0 else "+onepass" if args.hist == 0
                            else "+group" if args.group_attn > 0
                            else "+split" if args.group_attn == 0 else "")
    names = [n for n in args.configs.split(",") if n and n != this]
    if names:
        del step, inp, graph
        torch.cuda.empty_cache()
        result["configs"] = measure_configs(names, args.steps, args.warmup, torch)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
