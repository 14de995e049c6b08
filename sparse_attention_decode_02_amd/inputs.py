"""Seeded synthetic inputs for one paged DSA step.

This module draws random tensors and a random physical-page assignment with
the shapes and value distributions of the workloads, and does nothing else:
it holds none of the method's arithmetic (no scoring, selection, softmax or
row plan). Both the HIP path and the CPU oracle consume what it returns.

Workloads describe requests, not rows: request ``q`` has ``prior[q]`` tokens
already cached and appends ``new[q]`` tokens this step, all of whose keys,
values and indexer keys are in the caches when the step runs (a decode request
is ``new = 1``). How requests turn into rows is the row plan, which lives in
the library and, independently, in the oracle.

Value recipe (the same for every workload; see ``draw_values``):

* q, K, V ~ N(0, 1), drawn in fp32 and rounded to nearest-even bf16 for the
  bf16 workloads;
* indexer qI and kI are integers uniform in {-4, ..., 4}, stored exactly;
* the indexer head weights w are uniform over {0.5, 1, 2} per (row, head).

Small integers make every indexer dot product, ReLU, weighting and head sum
exact in fp32, so scores and the selection they decide have one right answer.

Page assignment: each request owns ceil((prior + new) / page) pages; the whole
pool is one random permutation, so logically adjacent pages of a request sit
at unrelated physical addresses. Unused block-table entries hold page 0.

Two generators: ``device="cpu"`` draws with NumPy's Philox (used for the small
workloads and every CPU test), ``device="cuda"`` draws with torch's device
generator so the multi-GiB caches of the large workloads never pass through
host memory. Each is deterministic for a given seed.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32" or "bf16": element type of q/K/V and of qI/kI
    page: int  # keys per page, shared by the indexer-key and K/V caches
    hq: int  # query heads
    hkv: int  # KV heads (one KV head per group of hq // hkv query heads)
    d: int  # attention head dim
    hi: int  # indexer query heads
    di: int  # indexer head dim (one indexer key head)
    topk: int
    prior: tuple  # tokens already cached, per request
    new: tuple  # tokens appended this step, per request
    seed: int = 0
    scale: float = field(default=float("nan"))  # attention scale; nan -> 1/sqrt(d)

    @property
    def num_reqs(self) -> int:
        return len(self.prior)

    @property
    def total_tokens(self) -> tuple:
        return tuple(p + n for p, n in zip(self.prior, self.new))

    @property
    def num_rows(self) -> int:
        return int(sum(self.new))

    @property
    def attn_scale(self) -> float:
        return 1.0 / math.sqrt(self.d) if math.isnan(self.scale) else self.scale

    def pages_per_req(self) -> list:
        return [-(-t // self.page) for t in self.total_tokens]

    @property
    def max_pages(self) -> int:
        return max(1, max(self.pages_per_req()))

    @property
    def num_pages(self) -> int:
        return max(1, sum(self.pages_per_req()))


def _decode(ctx):
    """Decode requests with the given context lengths (current token included)."""
    return tuple(c - 1 for c in ctx), tuple(1 for _ in ctx)


def tiny(seed: int = 20260001) -> Workload:
    """2 decode rows, contexts 37 and 100, page 16, 4 q / 1 KV head, d 64,
    indexer 4 x 32, top-k 16, fp32."""
    prior, new = _decode([37, 100])
    return Workload("tiny_f32", "f32", 16, 4, 1, 64, 4, 32, 16, prior, new, seed)


def decode(seed: int = 20260002) -> Workload:
    """Batch 8 at context 4096, page 64, 16 q / 2 KV heads, d 128, indexer
    64 x 128, top-k 2048, bf16."""
    prior, new = _decode([4096] * 8)
    return Workload("decode_b8_ctx4k_bf16", "bf16", 64, 16, 2, 128, 64, 128, 2048, prior, new, seed)


def headline(seed: int = 20260003) -> Workload:
    """Batch 64 at context 32768, page 64, 64 q / 8 KV heads, d 128, indexer
    64 x 128, top-k 2048, bf16."""
    prior, new = _decode([32768] * 64)
    return Workload("decode_b64_ctx32k_bf16", "bf16", 64, 64, 8, 128, 64, 128, 2048, prior, new, seed)


def long_context(seed: int = 20260006) -> Workload:
    """Long-context decode: batch 64, every context 204800 (the 200K decode
    point at which the pages quote their top-k stage), otherwise as the
    headline workload."""
    prior, new = _decode([204800] * 64)
    return Workload("decode_b64_ctx200k_bf16", "bf16", 64, 64, 8, 128, 64, 128, 2048, prior, new, seed)


def prefill_1m(seed: int = 20260007) -> Workload:
    """A 2048-token prefill chunk at 1M context: one request whose cache
    already holds 1048576 - 2048 tokens appends 2048 rows (causal lengths up
    to 1048576) -- the case whose full score buffer takes 8 GiB, the pages'
    reason for scoring in row windows; headline shapes otherwise."""
    return Workload("prefill_2048_ctx1m_bf16", "bf16", 64, 64, 8, 128, 64, 128, 2048,
                    (1048576 - 2048,), (2048,), seed)


def ragged_lengths(seed: int, batch: int = 64, lo_frac_rows: int = 6) -> list:
    """Context lengths for the ragged batch.

    ``lo_frac_rows`` rows (about 10% of 64) are log-uniform in [1, 2047] and
    the rest log-uniform in [2048, 65536]; one row is forced to 1 and one to
    65536; the order is shuffled by the seed.
    """
    rng = np.random.Generator(np.random.Philox(key=[seed, 0x52414744]))
    lo = np.exp(rng.uniform(math.log(1.0), math.log(2048.0), lo_frac_rows))
    hi = np.exp(rng.uniform(math.log(2048.0), math.log(65537.0), batch - lo_frac_rows))
    lo = np.clip(np.floor(lo), 1, 2047).astype(np.int64)
    hi = np.clip(np.floor(hi), 2048, 65536).astype(np.int64)
    lo[0] = 1
    hi[0] = 65536
    lens = np.concatenate([lo, hi])
    rng.shuffle(lens)
    return [int(x) for x in lens]


def ragged(seed: int = 20260004) -> Workload:
    """Batch 64, contexts per ``ragged_lengths``, page 64, 64 q / 8 KV heads,
    d 128, indexer 64 x 128, top-k 2048, bf16."""
    prior, new = _decode(ragged_lengths(seed))
    return Workload("ragged_b64_ctx1-64k_bf16", "bf16", 64, 64, 8, 128, 64, 128, 2048, prior, new, seed)


def mixed_lengths(seed: int, n_decode: int = 60, max_ctx: int = 131072) -> list:
    """Decode contexts for the mixed step: uniform integers in [1, max_ctx],
    one forced to max_ctx."""
    rng = np.random.Generator(np.random.Philox(key=[seed, 0x4D495844]))
    lens = rng.integers(1, max_ctx + 1, n_decode)
    lens[int(rng.integers(0, n_decode))] = max_ctx
    return [int(x) for x in lens]


def mixed(seed: int = 20260005) -> Workload:
    """4 chunked-prefill requests of 512 new tokens on prior contexts of 8192,
    then 60 decode requests at contexts up to 131072; 64 q / 8 KV heads, d 128,
    indexer 64 x 128, page 64, top-k 2048, bf16."""
    dec = mixed_lengths(seed)
    prior = tuple([8192] * 4 + [c - 1 for c in dec])
    new = tuple([512] * 4 + [1] * len(dec))
    return Workload("mixed_4x512pf_60dec_bf16", "bf16", 64, 64, 8, 128, 64, 128, 2048, prior, new, seed)


WORKLOADS = {
    "tiny": tiny,
    "decode": decode,
    "headline": headline,
    "long": long_context,
    "prefill_1m": prefill_1m,
    "ragged": ragged,
    "mixed": mixed,
}


def custom(base: Workload, **kw) -> Workload:
    """A copy of ``base`` with some fields replaced (prior/new as sequences)."""
    for key in ("prior", "new"):
        if key in kw:
            kw[key] = tuple(int(x) for x in kw[key])
    return replace(base, **kw)


# --------------------------------------------------------------------------
# Drawn tensors
# --------------------------------------------------------------------------


@dataclass
class StepInputs:
    """Every input of one step, as torch tensors on one device.

    Layouts (row-major, contiguous):
      qI        [rows][hi][di]            dtype
      w         [rows][hi]                float32
      q         [rows][hq][d]             dtype
      kI_cache  [num_pages][page][di]     dtype
      k_cache   [num_pages][page][hkv][d] dtype
      v_cache   [num_pages][page][hkv][d] dtype
      block_table [num_reqs][max_pages]   int32
    """

    wl: Workload
    qI: torch.Tensor
    w: torch.Tensor
    q: torch.Tensor
    kI_cache: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor

    @property
    def device(self):
        return self.q.device


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def page_assignment(wl: Workload) -> np.ndarray:
    """Block table: one random permutation of the physical page pool."""
    rng = np.random.Generator(np.random.Philox(key=[wl.seed, 0x50414745]))
    perm = rng.permutation(wl.num_pages).astype(np.int32)
    bt = np.zeros((wl.num_reqs, wl.max_pages), np.int32)
    off = 0
    for q, n in enumerate(wl.pages_per_req()):
        bt[q, :n] = perm[off:off + n]
        off += n
    return bt


def _host_draws(wl: Workload):
    rng = np.random.Generator(np.random.Philox(key=[wl.seed, 0x56414C53]))
    rows, P, npg = wl.num_rows, wl.page, wl.num_pages
    qI = rng.integers(-4, 5, (rows, wl.hi, wl.di)).astype(np.float32)
    w = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), (rows, wl.hi))
    q = rng.standard_normal((rows, wl.hq, wl.d), np.float32)
    kI = rng.integers(-4, 5, (npg, P, wl.di)).astype(np.float32)
    k = rng.standard_normal((npg, P, wl.hkv, wl.d), np.float32)
    v = rng.standard_normal((npg, P, wl.hkv, wl.d), np.float32)
    return qI, w, q, kI, k, v


def _device_normal(shape, gen, dt, device, chunk=1 << 27):
    out = torch.empty(shape, dtype=dt, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(dt)
    return out


def _device_int(shape, gen, dt, device, chunk=1 << 27):
    out = torch.empty(shape, dtype=dt, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randint(-4, 5, (e - s,), generator=gen, device=device, dtype=torch.int32).to(dt)
    return out


def generate(wl: Workload, device="cpu") -> StepInputs:
    """Draw every input of ``wl`` on ``device`` ("cpu" or a CUDA device)."""
    dev = torch.device(device)
    dt = torch_dtype(wl.dtype)
    bt = torch.from_numpy(page_assignment(wl)).to(dev)
    if dev.type == "cpu":
        qI, w, q, kI, k, v = _host_draws(wl)
        return StepInputs(
            wl,
            torch.from_numpy(qI).to(dt),
            torch.from_numpy(w),
            torch.from_numpy(q).to(dt),
            torch.from_numpy(kI).to(dt),
            torch.from_numpy(k).to(dt),
            torch.from_numpy(v).to(dt),
            bt,
        )
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(wl.seed))
    rows, P, npg = wl.num_rows, wl.page, wl.num_pages
    qI = _device_int((rows, wl.hi, wl.di), gen, dt, dev)
    widx = torch.randint(0, 3, (rows, wl.hi), generator=gen, device=dev)
    w = torch.tensor([0.5, 1.0, 2.0], device=dev)[widx].contiguous()
    q = _device_normal((rows, wl.hq, wl.d), gen, dt, dev)
    kI = _device_int((npg, P, wl.di), gen, dt, dev)
    k = _device_normal((npg, P, wl.hkv, wl.d), gen, dt, dev)
    v = _device_normal((npg, P, wl.hkv, wl.d), gen, dt, dev)
    return StepInputs(wl, qI, w, q, kI, k, v, bt)


def to_device(inp: StepInputs, device) -> StepInputs:
    """Copy every tensor of ``inp`` to ``device``."""
    return StepInputs(inp.wl, *(getattr(inp, f).to(device) for f in
                                ("qI", "w", "q", "kI_cache", "k_cache", "v_cache", "block_table")))


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Host float64 copy of a float tensor (bf16 widens exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()


def fill_uniform_ints(t: torch.Tensor, seed: int, lo: int, hi: int) -> torch.Tensor:
    """Overwrite ``t`` with integers uniform in [lo, hi] drawn from ``seed``
    (used by tests that need a different integer range)."""
    rng = np.random.Generator(np.random.Philox(key=[seed, 0x494E5453]))
    vals = rng.integers(lo, hi + 1, tuple(t.shape)).astype(np.float32)
    t.copy_(torch.from_numpy(vals).to(t.dtype))
    return t
