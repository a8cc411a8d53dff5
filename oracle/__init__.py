"""CPU oracle for MoE expert-parallel layout / scan / scatter / combine.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the package smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The product path (``permute_ep_layout_amd``) never
imports it, and the two share no code: the arithmetic lives in
``epl_oracle.c`` (plain single-threaded C), and this module only moves numpy
arrays in and out of it.

Each function cites, in ``epl_oracle.c``, the passage of the pages it
follows. Where no pin exists for a choice the function says so.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_ptr = ctypes.c_void_p

OK = 0
EINVAL = -1
ERANGE = -2


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed with oracle code {code}")
        self.code = code


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(rc, what)


class Oracle:
    """numpy front end of one build of ``epl_oracle.c`` (``path``)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.epl_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.epl_oracle_bf16_to_double.restype = ctypes.c_double
        lib.epl_oracle_bf16_from_double.argtypes = [ctypes.c_double]
        lib.epl_oracle_bf16_from_double.restype = ctypes.c_uint16
        lib.epl_oracle_layout.argtypes = [_c_i64, _c_i32, _c_i32, _c_i32, _ptr, _ptr, _ptr, _ptr]
        lib.epl_oracle_layout.restype = ctypes.c_int
        lib.epl_oracle_e4m3_from_double.argtypes = [ctypes.c_double]
        lib.epl_oracle_e4m3_from_double.restype = ctypes.c_uint8
        lib.epl_oracle_quantize_e4m3.argtypes = [_c_i64, _c_i32, _ptr, _ptr, _ptr]
        lib.epl_oracle_quantize_e4m3.restype = ctypes.c_int
        lib.epl_oracle_ll_dispatch.argtypes = [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                               _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                               _ptr]
        lib.epl_oracle_ll_dispatch.restype = ctypes.c_int
        lib.epl_oracle_rdma_counts.argtypes = [_c_i64, _c_i32, _c_i32, _ptr, _ptr]
        lib.epl_oracle_rdma_counts.restype = ctypes.c_int
        lib.epl_oracle_scan.argtypes = [_c_i32, _ptr, _c_i32, _ptr, _ptr]
        lib.epl_oracle_scan.restype = ctypes.c_int
        lib.epl_oracle_scatter.argtypes = [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _ptr, _ptr, _ptr, _ptr, _c_i64, _ptr, _ptr, _ptr, _ptr]
        lib.epl_oracle_scatter.restype = ctypes.c_int
        lib.epl_oracle_scatter_rows.argtypes = [_c_i64, _c_i32, _c_i32, _c_i64, _ptr, _c_i32,
                                                _c_i32, _ptr, _ptr, _ptr, _c_i64, _c_i64, _ptr,
                                                _ptr, _ptr, _ptr]
        lib.epl_oracle_scatter_rows.restype = ctypes.c_int
        lib.epl_oracle_expert_scale.argtypes = [_c_i64, _c_i32, _ptr, _ptr, _ptr]
        lib.epl_oracle_expert_scale.restype = ctypes.c_int
        lib.epl_oracle_combine.argtypes = [_c_i64, _c_i32, _c_i32, _ptr, _c_i64, _ptr, _ptr,
                                           _ptr, _c_i64, _ptr]
        lib.epl_oracle_combine.restype = ctypes.c_int
        lib.epl_oracle_time_pass.argtypes = [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _ptr,
                                             _c_i32, _c_i32, _ptr, _ptr, _ptr, _c_i32, _c_i64,
                                             _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                             _c_i32, _ptr, _ptr, _ptr]
        lib.epl_oracle_time_pass.restype = ctypes.c_int
        lib.epl_oracle_time_ll_pass.argtypes = [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                                _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                                _ptr, _ptr, _c_i64, _ptr, _ptr, _ptr, _ptr]
        lib.epl_oracle_time_ll_pass.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def bf16_to_double(self, bits: int) -> float:
        return float(self.lib.epl_oracle_bf16_to_double(int(bits)))

    def bf16_from_double(self, v: float) -> int:
        return int(self.lib.epl_oracle_bf16_from_double(float(v)))

    def bf16_from_double_array(self, v: np.ndarray) -> np.ndarray:
        f = self.lib.epl_oracle_bf16_from_double
        flat = np.asarray(v, dtype=np.float64).ravel()
        return np.array([f(float(a)) for a in flat], dtype=np.uint16).reshape(np.shape(v))

    def e4m3_from_double_array(self, v: np.ndarray) -> np.ndarray:
        f = self.lib.epl_oracle_e4m3_from_double
        flat = np.asarray(v, dtype=np.float64).ravel()
        return np.array([f(float(a)) for a in flat], dtype=np.uint8).reshape(np.shape(v))

    def quantize_e4m3(self, x: np.ndarray):
        """bf16 x [T, H] (uint16 bits) -> (e4m3 bytes [T, H], fp32 scales [T, H/128])."""
        xb = _c(x, np.uint16)
        T, H = xb.shape
        q = np.empty((T, H), np.uint8)
        sc = np.empty((T, H // 128), np.float32)
        _check(self.lib.epl_oracle_quantize_e4m3(T, H, _p(xb), _p(q), _p(sc)), "quantize_e4m3")
        return q, sc

    def ll_dispatch(self, x: Optional[np.ndarray], topk_idx: np.ndarray, num_experts: int,
                    tokens_per_segment: int, cap: int, hidden: Optional[int] = None):
        """Fixed-rectangle (low-latency) layout. Returns a dict with out
        [E, cap, H] u8 (rows past recv_count zero), out_scale [E, S, cap] f32,
        recv_count [E], src_info [E, cap] (-1 past recv_count), layout_range
        [E, T/M, 2] (begin, count), output_index [T, K] and overflow (bool).
        With x None only the indices are produced."""
        topk = _c(topk_idx, np.int64)
        T, K = topk.shape
        E, M = int(num_experts), int(tokens_per_segment)
        xb = None if x is None else _c(x, np.uint16)
        H = int(hidden) if xb is None else xb.shape[1]
        S = H // 128
        out = None if xb is None else np.zeros((E, cap, H), np.uint8)
        out_scale = None if xb is None else np.zeros((E, S, cap), np.float32)
        recv = np.empty(E, np.int32)
        src = np.full((E, cap), -1, np.int32)
        rng = np.empty((E, T // M if M else 0, 2), np.int32)
        oi = np.empty((T, K), np.int32)
        ovf = np.zeros(1, np.int32)
        _check(self.lib.epl_oracle_ll_dispatch(T, K, E, H, M, int(cap), _p(xb), _p(topk),
                                               _p(out), _p(out_scale), _p(recv), _p(src),
                                               _p(rng), _p(oi), _p(ovf)), "ll_dispatch")
        return dict(out=out, out_scale=out_scale, recv_count=recv, src_info=src,
                    layout_range=rng, output_index=oi, overflow=bool(ovf[0]))

    def layout(self, topk_idx: np.ndarray, num_experts: int, num_ranks: int):
        """Returns (num_tokens_per_expert [E] i32, num_tokens_per_rank [R] i32,
        is_token_in_rank [T, R] u8)."""
        topk = _c(topk_idx, np.int64)
        T, K = topk.shape
        cnt = np.empty(num_experts, np.int32)
        per_rank = np.empty(num_ranks, np.int32)
        in_rank = np.empty((T, num_ranks), np.uint8)
        _check(self.lib.epl_oracle_layout(T, K, num_experts, num_ranks, _p(topk), _p(cnt),
                                          _p(per_rank), _p(in_rank)), "layout")
        return cnt, per_rank, in_rank

    def rdma_counts(self, is_token_in_rank: np.ndarray, ranks_per_node: int):
        """num_tokens_per_rdma_rank [R / G] i32 for G = ranks_per_node GPUs
        per node, or None when all R ranks fit on one node (R <= G)."""
        in_rank = _c(is_token_in_rank, np.uint8)
        T, R = in_rank.shape
        G = int(ranks_per_node)
        if G <= 0 or G >= R:
            return None
        out = np.empty(R // G, np.int32)
        _check(self.lib.epl_oracle_rdma_counts(T, R, G, _p(in_rank), _p(out)), "rdma_counts")
        return out

    def scan(self, num_tokens_per_expert: np.ndarray, alignment: int = 0):
        """Returns (expert_start_loc [E] i32, total int); with alignment a > 1
        each expert's block is its count rounded up to a multiple of a."""
        cnt = _c(num_tokens_per_expert, np.int32)
        start = np.empty(cnt.size, np.int32)
        total = np.zeros(1, np.int64)
        _check(self.lib.epl_oracle_scan(cnt.size, _p(cnt), int(alignment), _p(start), _p(total)),
               "scan")
        return start, int(total[0])

    def scatter(self, x: Optional[np.ndarray], x_scale: Optional[np.ndarray],
                topk_idx: np.ndarray, expert_start_loc: np.ndarray, total: int,
                copy_rows: bool = True):
        """Returns (out [N, H] u16 or None, out_scale [N, S] f32 or None,
        m_indices [N] i32, output_index [T, K] i32). ``copy_rows=False``
        computes only the indices."""
        topk = _c(topk_idx, np.int64)
        T, K = topk.shape
        start = _c(expert_start_loc, np.int32)
        E = start.size
        H = int(x.shape[1]) if x is not None else 0
        S = int(x_scale.shape[1]) if x_scale is not None else 0
        xx = _c(x, np.uint16) if (x is not None and copy_rows) else None
        xs = _c(x_scale, np.float32) if (x_scale is not None and copy_rows) else None
        out = np.empty((total, H), np.uint16) if xx is not None else None
        out_scale = np.empty((total, S), np.float32) if xs is not None else None
        m_idx = np.empty(total, np.int32)
        oi = np.empty((T, K), np.int32)
        _check(self.lib.epl_oracle_scatter(T, K, E, H, S, _p(xx), _p(xs), _p(topk), _p(start),
                                           total, _p(out), _p(out_scale), _p(m_idx), _p(oi)),
               "scatter")
        return out, out_scale, m_idx, oi

    SCALE_NONE, SCALE_ROWS, SCALE_COLS = 0, 1, 2

    def scatter_rows(self, x_bytes: Optional[np.ndarray], x_scale_words: Optional[np.ndarray],
                     scale_format: int, topk_idx: np.ndarray, expert_start_loc: np.ndarray,
                     total: int, scale_ld: Optional[int] = None, copy_rows: bool = True):
        """Byte-row scatter (FP8 payload). x_bytes [T, B] uint8; x_scale_words
        [T, W] uint32. Returns (out [total, B] u8, out_scale, m_indices,
        output_index), out_scale being [total, W] (SCALE_ROWS) or the flat
        column-major buffer [W * scale_ld] (SCALE_COLS, default scale_ld = total)."""
        topk = _c(topk_idx, np.int64)
        T, K = topk.shape
        start = _c(expert_start_loc, np.int32)
        xb = None if x_bytes is None else _c(x_bytes, np.uint8)
        B = 0 if xb is None else xb.shape[1]
        xs = None if x_scale_words is None else _c(x_scale_words, np.uint32)
        W = 0 if xs is None else xs.shape[1]
        ld = total if scale_ld is None else int(scale_ld)
        out = np.empty((total, B), np.uint8) if (copy_rows and xb is not None) else None
        if xs is None or not copy_rows or scale_format == self.SCALE_NONE:
            out_scale = None
        elif scale_format == self.SCALE_ROWS:
            out_scale = np.empty((total, W), np.uint32)
        else:
            out_scale = np.empty(W * ld, np.uint32)
        m_idx = np.empty(total, np.int32)
        oi = np.empty((T, K), np.int32)
        _check(self.lib.epl_oracle_scatter_rows(T, K, start.size, B, _p(xb), int(scale_format), W,
                                                _p(xs), _p(topk), _p(start), total, ld,
                                                _p(out), _p(out_scale), _p(m_idx), _p(oi)),
               "scatter_rows")
        return out, out_scale, m_idx, oi

    def expert_scale(self, rows: np.ndarray, m_indices: np.ndarray) -> np.ndarray:
        """The large-batch workload's synthetic expert: bf16(row * (1 + e/256)).
        (Rows marked -1 are alignment padding; their output is not meaningful.)"""
        r = _c(rows, np.uint16)
        m = _c(m_indices, np.int32)
        N, H = r.shape
        out = np.empty_like(r)
        _check(self.lib.epl_oracle_expert_scale(N, H, _p(r), _p(m), _p(out)), "expert_scale")
        return out

    def combine(self, expert_out: np.ndarray, output_index: np.ndarray,
                topk_weights: np.ndarray, tokens: Optional[np.ndarray] = None) -> np.ndarray:
        """fp64 y [n, H] for the selected tokens (all tokens by default)."""
        eo = _c(expert_out, np.uint16)
        oi = _c(output_index, np.int32)
        w = _c(topk_weights, np.float32)
        T, K = oi.shape
        rows, H = eo.shape
        tk = None if tokens is None else _c(tokens, np.int64)
        n = T if tk is None else tk.size
        y = np.empty((n, H), np.float64)
        _check(self.lib.epl_oracle_combine(T, K, H, _p(eo), rows, _p(oi), _p(w), _p(tk), n,
                                           _p(y)), "combine")
        return y

    def timed_passes(self, x, x_scale, scale_format, topk_idx, topk_weights, num_experts,
                     num_ranks, hidden, expert_mode=0, expert_out=None, alignment=0):
        """A callable that runs one pass of layout, scan, byte-row scatter,
        (expert) and combine in the C timing harness on buffers allocated
        here once, and returns the step times in seconds. x is [T, row
        bytes] as uint8 (a bf16 array is viewed as bytes); x_scale [T, W]
        words or None; expert_mode 0 combines the scattered bf16 rows, 1
        applies the expert stand-in first, 2 combines ``expert_out``."""
        topk = _c(topk_idx, np.int64)
        T, K = topk.shape
        E, R, H = int(num_experts), int(num_ranks), int(hidden)
        xb = np.ascontiguousarray(x).view(np.uint8).reshape(T, -1)
        xs = None if x_scale is None else np.ascontiguousarray(x_scale).view(np.uint32)
        W = 0 if xs is None else xs.shape[1]
        fmt = int(scale_format) if xs is not None else self.SCALE_NONE
        w = _c(topk_weights, np.float32)
        a = max(int(alignment), 1)
        cap = -(-(int((topk >= 0).sum()) + E * (a - 1)) // a) * a    # rows always enough
        cnt, per_rank = np.empty(E, np.int32), np.empty(R, np.int32)
        in_rank, start = np.empty((T, R), np.uint8), np.empty(E, np.int32)
        out = np.empty((cap, xb.shape[1]), np.uint8)
        out_scale = None if xs is None else np.empty(cap * W, np.uint32)
        m_idx, oi = np.empty(cap, np.int32), np.empty((T, K), np.int32)
        eo = None
        if expert_mode == 1:
            eo = np.empty((cap, H), np.uint16)
        elif expert_mode == 2:
            eo = _c(expert_out, np.uint16)
        y = np.empty((T, H), np.float64)
        ns = np.zeros(5, np.int64)

        def run():
            _check(self.lib.epl_oracle_time_pass(
                T, K, E, R, H, xb.shape[1], _p(xb), fmt, W, _p(xs), _p(topk), _p(w),
                int(alignment), cap,
                _p(cnt), _p(per_rank), _p(in_rank), _p(start), _p(out), _p(out_scale),
                _p(m_idx), _p(oi), int(expert_mode), _p(eo), _p(y), _p(ns)), "time_pass")
            return dict(zip(("layout", "scan", "scatter", "expert", "combine"), ns * 1e-9))
        return run

    def timed_ll_passes(self, x, topk_idx, topk_weights, num_experts, tokens_per_segment, cap):
        """A callable that runs one pass of the low-latency dispatch and the
        combine over the experts' bf16 output rows in the C timing harness,
        on buffers allocated here once, and returns the step times in
        seconds. The expert output stands in as each placed row's bf16 token
        row, gathered compactly once (the placement is deterministic)."""
        xb = _c(x, np.uint16)
        topk = _c(topk_idx, np.int64)
        T, K = topk.shape
        H = xb.shape[1]
        E, M, cap = int(num_experts), int(tokens_per_segment), int(cap)
        S = H // 128
        out = np.empty((E, cap, H), np.uint8)          # only placed rows are touched
        out_scale = np.empty((E, S, cap), np.float32)
        recv = np.empty(E, np.int32)
        src = np.empty((E, cap), np.int32)
        rng = np.empty((E, T // M, 2), np.int32)
        oi = np.empty((T, K), np.int32)
        ovf = np.zeros(1, np.int32)
        first = self.ll_dispatch(None, topk, E, M, cap, hidden=H)["output_index"]
        valid = first >= 0
        compact = np.full(first.shape, -1, np.int32)
        compact[valid] = np.arange(int(valid.sum()), dtype=np.int32)
        eo = np.ascontiguousarray(np.repeat(xb, K, axis=0)[valid.ravel()])
        w = _c(topk_weights, np.float32)
        y = np.empty((T, H), np.float64)
        ns = np.zeros(2, np.int64)

        def run():
            _check(self.lib.epl_oracle_time_ll_pass(
                T, K, E, H, M, cap, _p(xb), _p(topk), _p(out), _p(out_scale), _p(recv), _p(src),
                _p(rng), _p(oi), _p(ovf), _p(eo), eo.shape[0], _p(compact), _p(w), _p(y),
                _p(ns)), "time_ll_pass")
            return dict(zip(("ll_dispatch", "combine"), ns * 1e-9))
        return run

    def run_all(self, x, x_scale, topk_idx, topk_weights, num_experts, num_ranks,
                expert_fn="identity", alignment=0):
        """The whole path on the CPU: layout, scan, scatter, (expert), combine."""
        cnt, per_rank, in_rank = self.layout(topk_idx, num_experts, num_ranks)
        start, total = self.scan(cnt, alignment)
        out, out_scale, m_idx, oi = self.scatter(x, x_scale, topk_idx, start, total)
        eo = out if expert_fn == "identity" else self.expert_scale(out, m_idx)
        y = self.combine(eo, oi, topk_weights)
        return dict(num_tokens_per_expert=cnt, num_tokens_per_rank=per_rank,
                    is_token_in_rank=in_rank, expert_start_loc=start, total=total,
                    out=out, out_scale=out_scale, m_indices=m_idx, output_index=oi,
                    expert_out=eo, y=y)


_DEFAULT = None


def default() -> Oracle:
    """The oracle built from ``epl_oracle.c`` (rebuilt when the source is newer),
    or the build named by EPL_ORACLE_LIB (the test suite's sanitizer run)."""
    global _DEFAULT
    if _DEFAULT is None:
        path, src = _build.LIB, _build.SRC
        if os.environ.get("EPL_ORACLE_LIB"):
            path = os.environ["EPL_ORACLE_LIB"]
        elif not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            _build.build()
        _DEFAULT = Oracle(path)
    return _DEFAULT


def lib_path() -> str:
    return _build.LIB


def __getattr__(name):
    # module-level shorthands: oracle.layout(...), oracle.scan(...), ...
    if name in ("bf16_to_double", "bf16_from_double", "bf16_from_double_array", "layout",
                "rdma_counts", "scan", "scatter", "expert_scale", "combine", "run_all",
                "e4m3_from_double_array", "quantize_e4m3", "ll_dispatch"):
        return getattr(default(), name)
    raise AttributeError(name)
