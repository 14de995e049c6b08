"""Python binding of libdsa.so: argument marshalling only.

Each function takes torch tensors, checks that they are contiguous, on the
GPU and of the expected dtype, and passes their data pointers, the sizes and
torch's current HIP stream to the C entry point of the same name; every step
of the computation runs in the library's HIP kernels. A negative status raises
``DsaError``. Importing this module loads the library and raises ImportError
when it has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m sparse_attention_decode_02_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_LL = ctypes.c_longlong
_IP = ctypes.POINTER(ctypes.c_int32)

F32, BF16 = 0, 1

_SIGS = {
    "dsa_status_string": (ctypes.c_char_p, [_I]),
    "dsa_abi_version": (_I, []),
    "dsa_plan_rows": (_I, [_I, _P, _P, _I, _P, _P, ctypes.POINTER(_I)]),
    "dsa_plan_blocks": (_I, [_I, _P, _I, _I, _P, ctypes.POINTER(_I)]),
    "dsa_score_width": (_I, [_I, _P, ctypes.POINTER(_I)]),
    "dsa_indexer_scores": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "dsa_indexer_scores_total": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                      _LL, _P]),
    "dsa_indexer_scores_hist": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                     _I, _LL, _P]),
    "dsa_score_hist": (_I, [_P, _P, _I, _I, _P, _P]),
    "dsa_topk_hist": (_I, [_P, _P, _P, _I, _I, _I, _LL, _P, _P]),
    "dsa_topk": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "dsa_topk_total": (_I, [_P, _P, _I, _I, _I, _LL, _P, _P]),
    "dsa_topk_chunked": (_I, [_P, _P, _I, _I, _I, _I, _P, _LL, _P, _P]),
    "dsa_topk_chunked_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "dsa_topk_chunked_slots": (_I, [_I, _I, _I, _I, ctypes.POINTER(_LL)]),
    "dsa_topk_chunk_suggest": (_I, [_I, _I, _I, _LL, ctypes.POINTER(_I)]),
    "dsa_indexer_topk_windowed": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                       _I, _I, _P, _LL, _I, _P, _LL, _P, _P]),
    "dsa_select_window_rows": (_I, [_I, _LL, ctypes.POINTER(_I)]),
    "dsa_read_probe": (_I, [_P, _LL, _P, _I, _P]),
    "dsa_sparse_attn": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _P]),
    "dsa_merge": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _I, _P]),
    "dsa_group_attn": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I,
                            _P]),
    "dsa_sparse_attn_splits": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_I)]),
    "dsa_sparse_attn_merged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _P]),
    "dsa_sparse_attn_merged_splits": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_I)]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_SIGS)


class DsaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def status_string(status: int) -> str:
    return _lib.dsa_status_string(int(status)).decode()


def abi_version() -> int:
    return _lib.dsa_abi_version()


def _check(fn, status):
    if status != 0:
        raise DsaError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Prepared:
    """One library call with its arguments checked and marshalled once
    (``prepare=True`` on a kernel wrapper); calling it with a stream (a torch
    stream, a raw hipStream_t as int, or None for torch's current stream)
    launches it. The tensors it was built from must stay alive and in place."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name, fn, args):
        self.name, self.fn, self.args, self.keep = name, fn, tuple(args), None

    def __call__(self, stream=None):
        status = self.fn(*self.args, _stream(stream))
        if status != 0:
            raise DsaError(self.name, status)


def _call(name, args, stream, prepare):
    fn = getattr(_lib, name)
    if prepare:
        return Prepared(name, fn, args)
    _check(name, fn(*args, _stream(stream)))
    return None


# --------------------------------------------------------------------------
# Row plan (host)
# --------------------------------------------------------------------------


def _host_i32(x):
    import numpy as np
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def plan_rows(prior, new):
    """(row_req, row_len) int32 NumPy arrays from dsa_plan_rows."""
    import numpy as np
    p, n = _host_i32(prior), _host_i32(new)
    if p.shape != n.shape:
        raise ValueError("prior and new differ in length")
    total = int(n.astype(np.int64).sum()) if n.size else 0
    req = np.zeros(max(total, 1), np.int32)
    ln = np.zeros(max(total, 1), np.int32)
    nr = _I(0)
    _check("dsa_plan_rows", _lib.dsa_plan_rows(len(p), p.ctypes.data, n.ctypes.data, total,
                                               req.ctypes.data, ln.ctypes.data, ctypes.byref(nr)))
    return req[: nr.value].copy(), ln[: nr.value].copy()


def plan_blocks(row_req, max_rows_per_block):
    """Score blocks int32 [num_blocks][2] (first_row, n_rows) from dsa_plan_blocks."""
    import numpy as np
    rq = _host_i32(row_req)
    blocks = np.zeros((max(len(rq), 1), 2), np.int32)
    nb = _I(0)
    _check("dsa_plan_blocks", _lib.dsa_plan_blocks(len(rq), rq.ctypes.data, int(max_rows_per_block),
                                                   len(blocks), blocks.ctypes.data, ctypes.byref(nb)))
    return blocks[: nb.value].copy()


def score_width(row_len) -> int:
    ln = _host_i32(row_len)
    w = _I(0)
    _check("dsa_score_width", _lib.dsa_score_width(len(ln), ln.ctypes.data, ctypes.byref(w)))
    return w.value


# --------------------------------------------------------------------------
# Kernels
# --------------------------------------------------------------------------


def indexer_scores(q_idx, w, k_idx_cache, block_table, row_req, row_len, scores, page_size,
                   blocks=None, stream=None, total_keys=None, prepare=False):
    """dsa_indexer_scores (dsa_indexer_scores_total when ``total_keys``, the
    host-known sum of the row lengths, is given): writes scores[r][:row_len[r]]
    in place."""
    rows, heads, dim = q_idx.shape
    dt = _dtype_code(q_idx)
    if k_idx_cache.dtype != q_idx.dtype:
        raise TypeError("q_idx and k_idx_cache dtypes differ")
    nb = 0 if blocks is None else int(blocks.shape[0])
    args = [_dev(q_idx, "q_idx"), _dev(w, "w", torch.float32), _dev(k_idx_cache, "k_idx_cache"),
            _dev(block_table, "block_table", torch.int32), _dev(row_req, "row_req", torch.int32),
            _dev(row_len, "row_len", torch.int32),
            None if blocks is None else _dev(blocks, "blocks", torch.int32), nb,
            _dev(scores, "scores", torch.float32), rows, int(scores.shape[1]), heads, dim,
            int(page_size), int(block_table.shape[1]), dt]
    if total_keys is None:
        p = _call("dsa_indexer_scores", args, stream, prepare)
    else:
        p = _call("dsa_indexer_scores_total", args + [int(total_keys)], stream, prepare)
    return p if prepare else scores


HIST_BINS = 4096  # bins of a score histogram: the top 12 bits of the order key


def indexer_scores_hist(q_idx, w, k_idx_cache, block_table, row_req, row_len, scores, hist,
                        page_size, blocks=None, stream=None, total_keys=0, prepare=False):
    """dsa_indexer_scores_hist: the scores, and each row's score histogram
    added to hist [rows][4096] uint32 (which must be zero on entry)."""
    rows, heads, dim = q_idx.shape
    dt = _dtype_code(q_idx)
    if k_idx_cache.dtype != q_idx.dtype:
        raise TypeError("q_idx and k_idx_cache dtypes differ")
    if hist.dtype != torch.int32 and hist.dtype != torch.uint32:
        raise TypeError("hist must be a 32-bit integer tensor")
    nb = 0 if blocks is None else int(blocks.shape[0])
    p = _call("dsa_indexer_scores_hist", [
        _dev(q_idx, "q_idx"), _dev(w, "w", torch.float32), _dev(k_idx_cache, "k_idx_cache"),
        _dev(block_table, "block_table", torch.int32), _dev(row_req, "row_req", torch.int32),
        _dev(row_len, "row_len", torch.int32),
        None if blocks is None else _dev(blocks, "blocks", torch.int32), nb,
        _dev(scores, "scores", torch.float32), _dev(hist, "hist"), rows, int(scores.shape[1]),
        heads, dim, int(page_size), int(block_table.shape[1]), dt, int(total_keys)], stream, prepare)
    return p if prepare else scores


def score_hist(scores, row_len, hist, stream=None):
    """dsa_score_hist: hist [rows][4096] of the scores already written."""
    rows, width = scores.shape
    _call("dsa_score_hist", [_dev(scores, "scores", torch.float32),
                             _dev(row_len, "row_len", torch.int32), rows, width,
                             _dev(hist, "hist")], stream, False)
    return hist


def topk_hist(scores, row_len, hist, k, idx, stream=None, total_keys=0, prepare=False):
    """dsa_topk_hist: dsa_topk from the rows' score histograms (hist is left
    zero); writes idx [rows][k] in place."""
    rows, width = scores.shape
    p = _call("dsa_topk_hist", [
        _dev(scores, "scores", torch.float32), _dev(row_len, "row_len", torch.int32),
        _dev(hist, "hist"), rows, width, int(k), int(total_keys), _dev(idx, "idx", torch.int32)],
        stream, prepare)
    return p if prepare else idx


def topk(scores, row_len, k, idx, stream=None, total_keys=None, prepare=False):
    """dsa_topk (dsa_topk_total when ``total_keys``, the host-known sum of the
    row lengths, is given): writes idx [rows][k] in place."""
    rows, width = scores.shape
    args = [_dev(scores, "scores", torch.float32), _dev(row_len, "row_len", torch.int32), rows,
            width, int(k)]
    if total_keys is None:
        p = _call("dsa_topk", args + [_dev(idx, "idx", torch.int32)], stream, prepare)
    else:
        p = _call("dsa_topk_total", args + [int(total_keys), _dev(idx, "idx", torch.int32)],
                  stream, prepare)
    return p if prepare else idx


def topk_chunked_slots(rows, width, k, chunk) -> int:
    """dsa_topk_chunked_slots: int32 candidate slots dsa_topk_chunked needs."""
    out = _LL(0)
    _check("dsa_topk_chunked_slots", _lib.dsa_topk_chunked_slots(
        int(rows), int(width), int(k), int(chunk), ctypes.byref(out)))
    return out.value


def topk_chunked(scores, row_len, k, chunk, cand, idx, stream=None, prepare=False):
    """dsa_topk_chunked: the dsa_topk result in two stages (segment winners in
    cand, then each row's top-k among them); writes idx [rows][k] in place."""
    rows, width = scores.shape
    p = _call("dsa_topk_chunked", [
        _dev(scores, "scores", torch.float32), _dev(row_len, "row_len", torch.int32), rows, width,
        int(k), int(chunk), _dev(cand, "cand", torch.int32), int(cand.numel()),
        _dev(idx, "idx", torch.int32)], stream, prepare)
    return p if prepare else idx


TOPK_NOALLOC_MAX_SLOTS = 1 << 22  # DSA_TOPK_NOALLOC_MAX_SLOTS


def topk_chunked_noalloc(scores, row_len, k, chunk, idx, stream=None, prepare=False):
    """dsa_topk_chunked_noalloc: dsa_topk_chunked with the library's own fixed
    candidate workspace (no allocation; calls on one device must not overlap)."""
    rows, width = scores.shape
    p = _call("dsa_topk_chunked_noalloc", [
        _dev(scores, "scores", torch.float32), _dev(row_len, "row_len", torch.int32), rows, width,
        int(k), int(chunk), _dev(idx, "idx", torch.int32)], stream, prepare)
    return p if prepare else idx


def topk_chunk_suggest(rows, width, k, total_keys=0) -> int:
    """dsa_topk_chunk_suggest: segment length for dsa_topk_chunked, or 0 for
    dsa_topk (total_keys: the sum of the row lengths, 0 if unknown)."""
    out = _I(0)
    _check("dsa_topk_chunk_suggest", _lib.dsa_topk_chunk_suggest(
        int(rows), int(width), int(k), int(total_keys), ctypes.byref(out)))
    return out.value


def select_window_rows(width, score_buffer_bytes) -> int:
    """dsa_select_window_rows: rows per window for a score buffer of this size."""
    out = _I(0)
    _check("dsa_select_window_rows", _lib.dsa_select_window_rows(
        int(width), int(score_buffer_bytes), ctypes.byref(out)))
    return out.value


def indexer_topk_windowed(q_idx, w, k_idx_cache, block_table, row_req, row_len, width, page_size,
                          k, score_buffer, idx, topk_chunk=0, cand=None, stream=None,
                          prepare=False, blocks=None, blocks_host=None):
    """dsa_indexer_topk_windowed: scores and top-k of every row, a window of
    rows at a time through score_buffer (any float32 device tensor; its byte
    size sets the window); optional score blocks as a device tensor plus the
    same plan on the host (NumPy); writes idx [rows][k] in place."""
    import numpy as np
    nb = 0
    bh = None
    if blocks is not None:
        bh = np.ascontiguousarray(np.asarray(blocks_host, dtype=np.int32))
        nb = int(bh.shape[0])
        if tuple(blocks.shape) != tuple(bh.shape):
            raise ValueError("blocks and blocks_host differ")
    rows, heads, dim = q_idx.shape
    if k_idx_cache.dtype != q_idx.dtype:
        raise TypeError("q_idx and k_idx_cache dtypes differ")
    p = _call("dsa_indexer_topk_windowed", [
        _dev(q_idx, "q_idx"), _dev(w, "w", torch.float32), _dev(k_idx_cache, "k_idx_cache"),
        _dev(block_table, "block_table", torch.int32), _dev(row_req, "row_req", torch.int32),
        _dev(row_len, "row_len", torch.int32), None if bh is None else bh.ctypes.data,
        None if blocks is None else _dev(blocks, "blocks", torch.int32), nb,
        rows, int(width), heads, dim, int(page_size),
        int(block_table.shape[1]), _dtype_code(q_idx), int(k),
        _dev(score_buffer, "score_buffer", torch.float32), int(score_buffer.numel()) * 4,
        int(topk_chunk), None if cand is None else _dev(cand, "cand", torch.int32),
        0 if cand is None else int(cand.numel()), _dev(idx, "idx", torch.int32)], stream, prepare)
    if prepare:
        p.keep = bh  # the host plan must outlive the prepared call
    return p if prepare else idx


def sparse_attn(q, k_cache, v_cache, block_table, row_req, idx, page_size, scale, num_splits,
                part_o, part_lse, stream=None, prepare=False):
    """dsa_sparse_attn: writes part_o [rows][Hq][S][d] and part_lse [rows][Hq][S]."""
    rows, hq, d = q.shape
    hkv = k_cache.shape[2]
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache dtypes differ")
    p = _call("dsa_sparse_attn", [
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32), _dev(row_req, "row_req", torch.int32),
        _dev(idx, "idx", torch.int32), rows, hq, hkv, d, int(idx.shape[1]), int(page_size),
        int(block_table.shape[1]), float(scale), int(num_splits),
        _dev(part_o, "part_o", torch.float32), _dev(part_lse, "part_lse", torch.float32), dt],
        stream, prepare)
    return p if prepare else (part_o, part_lse)


def group_attn(q, k_cache, v_cache, block_table, row_req, idx, groups, page_size, scale, out,
               out_lse=None, stream=None, prepare=False):
    """dsa_group_attn: attention of the rows of each group [first_row, n_rows]
    over the union of their selections; writes out (and out_lse) in place."""
    rows, hq, d = q.shape
    hkv = k_cache.shape[2]
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k_cache, v_cache and out dtypes differ")
    p = _call("dsa_group_attn", [
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32), _dev(row_req, "row_req", torch.int32),
        _dev(idx, "idx", torch.int32), _dev(groups, "groups", torch.int32), int(groups.shape[0]),
        rows, hq, hkv, d, int(idx.shape[1]), int(page_size), int(block_table.shape[1]),
        float(scale), _dev(out, "out"),
        None if out_lse is None else _dev(out_lse, "out_lse", torch.float32), dt], stream, prepare)
    return p if prepare else out


def sparse_attn_splits(rows, num_q_heads, num_kv_heads, head_dim, k, dtype) -> int:
    """dsa_sparse_attn_splits: the split count that fills the current device."""
    code = BF16 if dtype == torch.bfloat16 else F32 if dtype == torch.float32 else -1
    out = _I(0)
    _check("dsa_sparse_attn_splits", _lib.dsa_sparse_attn_splits(
        int(rows), int(num_q_heads), int(num_kv_heads), int(head_dim), int(k), code,
        ctypes.byref(out)))
    return out.value


def sparse_attn_merged(q, k_cache, v_cache, block_table, row_req, idx, page_size, scale,
                       num_splits, out, out_lse=None, stream=None, prepare=False):
    """dsa_sparse_attn_merged: attention and merge in one launch; writes out
    [rows][Hq][d] (and out_lse [rows][Hq] if given)."""
    rows, hq, d = q.shape
    hkv = k_cache.shape[2]
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k_cache, v_cache and out dtypes differ")
    p = _call("dsa_sparse_attn_merged", [
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32), _dev(row_req, "row_req", torch.int32),
        _dev(idx, "idx", torch.int32), rows, hq, hkv, d, int(idx.shape[1]), int(page_size),
        int(block_table.shape[1]), float(scale), int(num_splits), _dev(out, "out"),
        None if out_lse is None else _dev(out_lse, "out_lse", torch.float32), dt], stream, prepare)
    return p if prepare else (out, out_lse)


def sparse_attn_merged_splits(rows, num_q_heads, num_kv_heads, head_dim, k, dtype) -> int:
    """dsa_sparse_attn_merged_splits: the split count for dsa_sparse_attn_merged."""
    code = BF16 if dtype == torch.bfloat16 else F32 if dtype == torch.float32 else -1
    out = _I(0)
    _check("dsa_sparse_attn_merged_splits", _lib.dsa_sparse_attn_merged_splits(
        int(rows), int(num_q_heads), int(num_kv_heads), int(head_dim), int(k), code,
        ctypes.byref(out)))
    return out.value


def merge(part_o, part_lse, out, out_lse=None, stream=None, prepare=False):
    """dsa_merge: writes out [rows][Hq][d] (and out_lse [rows][Hq] if given)."""
    rows, hq, S, d = part_o.shape
    p = _call("dsa_merge", [
        _dev(part_o, "part_o", torch.float32), _dev(part_lse, "part_lse", torch.float32), rows, hq,
        d, S, _dev(out, "out"), None if out_lse is None else _dev(out_lse, "out_lse", torch.float32),
        _dtype_code(out)], stream, prepare)
    return p if prepare else (out, out_lse)


def read_probe(src, sink, stream=None):
    """dsa_read_probe: one streaming read of ``src`` (per-workgroup sums into sink)."""
    _check("dsa_read_probe", _lib.dsa_read_probe(
        _dev(src, "src"), int(src.numel() * src.element_size()), _dev(sink, "sink", torch.float32),
        int(sink.numel()), _stream(stream)))
    return sink
