"""Python binding of libidx.so, the MI355X (gfx950) DSA lightning-indexer top-k.

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  If the library has
not been built, every entry point raises (there is no CPU fallback).

Entry points (same names as the C ABI in include/idx.h):
    idx_score(prob, out=None, ld=None)        -> fp32 [rows, ld] materialised scores
    idx_select(scores, length, k, ...)        -> int32 [rows, k] exact top-k
    idx_fused_topk(prob, k, ...)              -> int32 [rows, k] (+ stats dict)
    idx_fused_workspace(prob, k), idx_select_workspace(rows, ld, k), idx_row_split(...)
``DeviceProblem.from_host(workloads.Problem)`` uploads a host problem.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libidx.so")

IDX_OK, IDX_EINVAL, IDX_EFMT, IDX_EALIGN, IDX_EWS, IDX_EHIP, IDX_ENODEV, IDX_ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
IDX_NOALLOC_SCRATCH_BYTES = 128 << 20
IDX_FMT_E4M3, IDX_FMT_MXFP4 = 1, 2
IDX_HEAD_DIM, IDX_MAX_TOPK, IDX_PAGE = 128, 2048, 64

_c_p = ctypes.c_void_p


class IdxDebug(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int32), ("threshold_mode", ctypes.c_int32),
                ("threshold_row_mod", ctypes.c_int32), ("tie_cap", ctypes.c_int32)]


class IdxProblem(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("fmt", ctypes.c_int32),
        ("q", _c_p), ("q_sf", _c_p), ("k", _c_p), ("k_sf", _c_p), ("k_scale", _c_p), ("w", _c_p),
        ("ks", _c_p), ("ke", _c_p), ("num_keys", ctypes.c_int64), ("page_table", _c_p), ("row_req", _c_p),
        ("num_req", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("debug", ctypes.POINTER(IdxDebug)),
    ]


class IdxStats(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("rows_store_all", ctypes.c_int32), ("rows_sampled", ctypes.c_int32),
        ("fallback_rows", ctypes.c_int32), ("max_count", ctypes.c_int32), ("min_count", ctypes.c_int32),
        ("total_count", ctypes.c_int64), ("cap", ctypes.c_int32), ("sample_stride", ctypes.c_int32),
        ("sample_keys", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class IdxError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {_lib().idx_strerror(code).decode()} ({code})")


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sparse_attention_indexer_score_amd.build` "
                               "(there is no CPU fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER(IdxProblem)
        sig = {
            "idx_score": (ctypes.c_int, [P, _c_p, i64, _c_p, sz, _c_p]),
            "idx_score_workspace": (sz, [P]),
            "idx_select": (ctypes.c_int, [_c_p, i64, _c_p, _c_p, i32, i32, _c_p, _c_p, sz, _c_p]),
            "idx_select_split": (ctypes.c_int, [_c_p, i64, _c_p, _c_p, i32, i32, _c_p, _c_p, sz, i32, _c_p]),
            "idx_row_split": (i32, [i32, i64, i32]),
            "idx_select_workspace": (sz, [i32, i64, i32]),
            "idx_fused_topk": (ctypes.c_int, [P, i32, _c_p, _c_p, sz, ctypes.POINTER(IdxStats), _c_p]),
            "idx_fused_workspace": (sz, [P, i32]),
            "idx_fused_topk_noalloc": (ctypes.c_int, [P, i32, _c_p, _c_p]),
            "idx_page_slots": (ctypes.c_int, [_c_p, i32, i32, _c_p, _c_p, _c_p, i32, _c_p, _c_p]),
            "idx_sparse_attn": (ctypes.c_int, [_c_p, _c_p, _c_p, i64, _c_p, i32, i32, i32, i32, ctypes.c_float,
                                               ctypes.c_float, _c_p, _c_p]),
            "idx_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "idx_version": (i32, []),
            "idx_timing_enable": (ctypes.c_int, [i32]),
            "idx_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), i32]),
            "idx_timing_disable": (ctypes.c_int, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(code: int, what: str):
    if code != IDX_OK:
        raise IdxError(code, what)


def _workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled uint8 device buffer whose data pointer is 256-byte aligned (the selection's
    row-split counters then start at the value every call leaves them at)."""
    if nbytes == 0:
        return torch.empty(0, dtype=torch.uint8, device=device)
    buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


class DeviceProblem:
    """Device-resident indexer problem (torch tensors) plus the scalar fields of idx_problem."""

    def __init__(self, fmt: int, rows: int, heads: int, q, q_sf, k, k_sf, k_scale, w, ks, ke, num_keys: int,
                 page_table=None, row_req=None, num_req: int = 0, max_pages: int = 0):
        self.fmt, self.rows, self.heads = fmt, rows, heads
        self.q, self.q_sf, self.k, self.k_sf, self.k_scale = q, q_sf, k, k_sf, k_scale
        self.w, self.ks, self.ke = w, ks, ke
        self.num_keys = num_keys
        self.page_table, self.row_req = page_table, row_req
        self.num_req, self.max_pages = num_req, max_pages
        self.debug: Optional[IdxDebug] = None

    @classmethod
    def from_host(cls, p, device="cuda") -> "DeviceProblem":
        def up(a, dtype=None):
            if a is None:
                return None
            t = torch.from_numpy(a.copy() if not a.flags.c_contiguous else a)
            if dtype is not None:
                t = t.view(dtype)
            return t.to(device, non_blocking=False)
        fmt = IDX_FMT_E4M3 if p.fmt == "e4m3" else IDX_FMT_MXFP4
        num_req = 0 if p.page_table is None else p.page_table.shape[0]
        max_pages = 0 if p.page_table is None else p.page_table.shape[1]
        return cls(fmt, p.rows, p.heads, up(p.q), up(p.q_sf), up(p.k), up(p.k_sf), up(p.k_scale),
                   up(p.w.view("int16"), None), up(p.ks), up(p.ke), p.num_keys, up(p.page_table), up(p.row_req),
                   num_req, max_pages)

    def rows_slice(self, r0: int, r1: int) -> "DeviceProblem":
        """Rows [r0, r1) sharing the same keys (views, no copy)."""
        def sl(t):
            return None if t is None else t[r0:r1]
        d = DeviceProblem(self.fmt, r1 - r0, self.heads, sl(self.q), sl(self.q_sf), self.k, self.k_sf,
                          self.k_scale, sl(self.w), sl(self.ks), sl(self.ke), self.num_keys, self.page_table,
                          sl(self.row_req), self.num_req, self.max_pages)
        d.debug = self.debug
        return d

    @property
    def device(self):
        return self.q.device

    def struct(self) -> IdxProblem:
        s = IdxProblem()
        s.rows, s.heads, s.head_dim, s.fmt = self.rows, self.heads, IDX_HEAD_DIM, self.fmt
        s.q, s.q_sf, s.k, s.k_sf = _ptr(self.q), _ptr(self.q_sf), _ptr(self.k), _ptr(self.k_sf)
        s.k_scale, s.w, s.ks, s.ke = _ptr(self.k_scale), _ptr(self.w), _ptr(self.ks), _ptr(self.ke)
        s.num_keys = self.num_keys
        s.page_table, s.row_req = _ptr(self.page_table), _ptr(self.row_req)
        s.num_req, s.max_pages = self.num_req, self.max_pages
        if self.debug is not None:
            s.debug = ctypes.pointer(self.debug)
        return s

    def key_span(self) -> int:
        return self.max_pages * IDX_PAGE if self.page_table is not None else self.num_keys


# ----------------------------------------------------------------------------- scoring

def idx_score_workspace(prob: DeviceProblem) -> int:
    s = prob.struct()
    return int(_lib().idx_score_workspace(ctypes.byref(s)))


def idx_score(prob: DeviceProblem, out: Optional[torch.Tensor] = None, ld: Optional[int] = None,
              stream=None) -> torch.Tensor:
    """Materialised fp32 scores: out[r, s - ks[r]] for every visible key (other entries untouched)."""
    if ld is None:
        ld = out.shape[1] if out is not None else max(1, int((prob.ke - prob.ks).max().item()) if prob.rows else 1)
    if out is None:
        out = torch.full((prob.rows, ld), float("nan"), dtype=torch.float32, device=prob.device)
    s = prob.struct()
    nb = int(_lib().idx_score_workspace(ctypes.byref(s)))
    ws = _workspace(nb, prob.device)
    _check(_lib().idx_score(ctypes.byref(s), _ptr(out), ld, _ptr(ws) if nb else None, nb, _stream(stream)),
           "idx_score")
    return out


# ----------------------------------------------------------------------------- selection

def idx_select_workspace(rows: int, ld: int, k: int) -> int:
    return int(_lib().idx_select_workspace(rows, ld, k))


def idx_row_split(rows: int, row_len: int, cu_count: int) -> int:
    return int(_lib().idx_row_split(rows, row_len, cu_count))


def idx_select(scores: torch.Tensor, length: torch.Tensor, k: int, row_start: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, split: Optional[int] = None, stream=None,
               workspace: bool = True) -> torch.Tensor:
    """Exact top-k of each row of scores[rows, ld] (row r: scores[r, row_start[r] + j], j < length[r]).
    workspace=False passes no workspace (the row split is then off: one workgroup per row)."""
    assert scores.dtype == torch.float32 and scores.dim() == 2 and scores.is_contiguous()
    rows, ld = scores.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    nb = idx_select_workspace(rows, ld, k) if workspace else 0
    ws = _workspace(nb, scores.device) if workspace else None
    L = _lib()
    if split is None:
        rc = L.idx_select(_ptr(scores), ld, _ptr(row_start), _ptr(length), rows, k, _ptr(out), _ptr(ws), nb,
                          _stream(stream))
    else:
        rc = L.idx_select_split(_ptr(scores), ld, _ptr(row_start), _ptr(length), rows, k, _ptr(out), _ptr(ws), nb,
                                split, _stream(stream))
    _check(rc, "idx_select")
    return out


class SelectRunner:
    """idx_select with a preallocated workspace and output (repeated calls allocate nothing)."""

    def __init__(self, scores: torch.Tensor, length: torch.Tensor, k: int, row_start: Optional[torch.Tensor] = None,
                 split: Optional[int] = None):
        assert scores.dtype == torch.float32 and scores.dim() == 2 and scores.is_contiguous()
        self.scores, self.length, self.k, self.row_start, self.split = scores, length, k, row_start, split
        rows, ld = scores.shape
        self.rows, self.ld = rows, ld
        self.nbytes = idx_select_workspace(rows, ld, k)
        self.ws = _workspace(self.nbytes, scores.device)
        self.out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)

    def __call__(self, stream=None) -> torch.Tensor:
        L = _lib()
        if self.split is None:
            rc = L.idx_select(_ptr(self.scores), self.ld, _ptr(self.row_start), _ptr(self.length), self.rows, self.k,
                              _ptr(self.out), _ptr(self.ws), self.nbytes, _stream(stream))
        else:
            rc = L.idx_select_split(_ptr(self.scores), self.ld, _ptr(self.row_start), _ptr(self.length), self.rows,
                                    self.k, _ptr(self.out), _ptr(self.ws), self.nbytes, self.split, _stream(stream))
        _check(rc, "idx_select")
        return self.out


class ScoreRunner:
    """idx_score into a preallocated [rows, ld] buffer with a preallocated workspace."""

    def __init__(self, prob: DeviceProblem, ld: Optional[int] = None):
        self.prob = prob
        self.s = prob.struct()
        self.ld = ld if ld is not None else max(1, int((prob.ke - prob.ks).max().item()) if prob.rows else 1)
        self.out = torch.empty((prob.rows, self.ld), dtype=torch.float32, device=prob.device)
        self.nbytes = idx_score_workspace(prob)
        self.ws = _workspace(self.nbytes, prob.device)

    def __call__(self, stream=None) -> torch.Tensor:
        _check(_lib().idx_score(ctypes.byref(self.s), _ptr(self.out), self.ld, _ptr(self.ws) if self.nbytes else None,
                                self.nbytes, _stream(stream)), "idx_score")
        return self.out


# ----------------------------------------------------------------------------- fused top-k

def idx_fused_workspace(prob: DeviceProblem, k: int) -> int:
    s = prob.struct()
    return int(_lib().idx_fused_workspace(ctypes.byref(s), k))


class FusedRunner:
    """Holds a workspace so repeated calls allocate nothing (used by the benchmark)."""

    def __init__(self, prob: DeviceProblem, k: int):
        self.prob, self.k = prob, k
        self.s = prob.struct()
        self.nbytes = idx_fused_workspace(prob, k)
        if self.nbytes == 0 and prob.rows > 0:
            raise IdxError(IDX_EINVAL, "idx_fused_workspace")
        self.ws = _workspace(self.nbytes, prob.device)
        self.out = torch.empty((prob.rows, k), dtype=torch.int32, device=prob.device)

    def __call__(self, stats: bool = False, stream=None):
        st = IdxStats() if stats else None
        rc = _lib().idx_fused_topk(ctypes.byref(self.s), self.k, _ptr(self.out), _ptr(self.ws), self.nbytes,
                                   ctypes.byref(st) if st is not None else None, _stream(stream))
        _check(rc, "idx_fused_topk")
        return self.out, (_stats_dict(st) if st is not None else None)


def _stats_dict(st: IdxStats) -> dict:
    return {name: getattr(st, name) for name, _ in IdxStats._fields_ if name != "reserved"}


def idx_fused_topk(prob: DeviceProblem, k: int, stats: bool = False, stream=None):
    """Exact top-k without materialising scores.  Returns out [rows, k] (and a stats dict)."""
    out, st = FusedRunner(prob, k)(stats=stats, stream=stream)
    return (out, st) if stats else out


def idx_fused_topk_noalloc(prob: DeviceProblem, k: int, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """idx_fused_topk on the library's fixed scratch (no workspace argument).  out: int32
    [rows, k] (allocated here when not given)."""
    if out is None:
        out = torch.empty((prob.rows, k), dtype=torch.int32, device=prob.device)
    s = prob.struct()
    _check(_lib().idx_fused_topk_noalloc(ctypes.byref(s), k, _ptr(out), _stream(stream)), "idx_fused_topk_noalloc")
    return out


def idx_page_slots(idx: torch.Tensor, page_table: torch.Tensor, row_req: torch.Tensor,
                   ks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Physical KV slots of selected positions: out[r, j] = page_table[row_req[r], p // 64] * 64 + p % 64
    with p = ks[r] + idx[r, j] (ks None: 0); -1 entries stay -1.  out may be idx (in place)."""
    assert idx.dtype == torch.int32 and idx.dim() == 2 and idx.is_contiguous()
    rows, k = idx.shape
    if out is None:
        out = torch.empty_like(idx)
    _check(_lib().idx_page_slots(_ptr(idx), rows, k, _ptr(ks), _ptr(page_table), _ptr(row_req),
                                 page_table.shape[1], _ptr(out), _stream(stream)), "idx_page_slots")
    return out


def idx_sparse_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, slots: torch.Tensor,
                    softmax_scale: float, output_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Attention of each query row over its selected KV slots (the top-k's consumer).
    q: bf16 bit patterns [rows, hq, 128] (int16/uint16 or bfloat16); k_cache, v_cache: e4m3 bytes
    [num_slots, hkv, 128] (uint8); slots: int32 [rows, width], entries outside [0, num_slots)
    ignored.  Returns fp32 [rows, hq, 128]."""
    assert q.dim() == 3 and q.shape[2] == 128 and q.element_size() == 2 and q.is_contiguous()
    assert k_cache.dtype == torch.uint8 and k_cache.dim() == 3 and k_cache.is_contiguous()
    assert v_cache.shape == k_cache.shape and v_cache.dtype == torch.uint8 and v_cache.is_contiguous()
    assert slots.dtype == torch.int32 and slots.dim() == 2 and slots.is_contiguous()
    rows, hq, _ = q.shape
    num_slots, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty((rows, hq, 128), dtype=torch.float32, device=q.device)
    _check(_lib().idx_sparse_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), num_slots, _ptr(slots), rows, hq, hkv,
                                  slots.shape[1], float(softmax_scale), float(output_scale), _ptr(out),
                                  _stream(stream)), "idx_sparse_attn")
    return out


def version() -> int:
    return int(_lib().idx_version())


FUSED_STAGES = ("sample", "threshold", "score_filter", "slab_select", "fallback")


def idx_timing_enable(max_calls: int):
    _check(_lib().idx_timing_enable(max_calls), "idx_timing_enable")


def idx_timing_read(max_calls: int):
    """Per timed idx_fused_topk call, the milliseconds of its five stages (list of dicts)."""
    buf = (ctypes.c_float * (5 * max_calls))()
    n = _lib().idx_timing_read(buf, max_calls)
    if n < 0:
        raise IdxError(n, "idx_timing_read")
    return [dict(zip(FUSED_STAGES, buf[5 * c:5 * c + 5])) for c in range(n)]


def idx_timing_disable():
    _check(_lib().idx_timing_disable(), "idx_timing_disable")
