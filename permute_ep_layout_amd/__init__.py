"""MoE expert-parallel layout / dispatch / combine on one MI355X rank.

Thin Python binding of ``libepl.so`` (C ABI in ``include/epl.h``). The
functions named ``epl_*`` mirror the C entry points one to one and do only
argument marshalling: they check tensor dtypes, shapes and devices, pass raw
pointers and the current HIP stream, and turn status codes into exceptions.
Every step of the path runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and using the package without the built library raises.

``dispatch`` and ``combine`` are tensor-level conveniences on top of them:
they allocate outputs with ``torch.empty`` and call the same entry points.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

from . import build as _build

__all__ = [
    "EplError", "Problem", "lib_path", "load", "is_built", "ensure_built",
    "epl_validate", "epl_workspace_bytes", "epl_capacity_rows", "epl_layout", "epl_scan",
    "epl_scatter", "epl_dispatch", "epl_combine", "epl_expert_scale", "epl_status", "epl_total",
    "epl_strerror", "epl_version", "dispatch", "combine", "expert_scale", "DispatchResult",
    "EPL_OK", "EPL_EINVAL", "EPL_ERANGE", "EPL_ECAPACITY", "EPL_EHIP", "EPL_OUT_F32",
    "EPL_OUT_BF16", "prepare", "epl_scatter_fp8", "epl_dispatch_fp8", "EPL_SCALE_NONE",
    "EPL_SCALE_F32", "EPL_SCALE_UE8M0", "epl_dispatch_static", "StaticWorkspace",
    "EPL_STATIC_WORKSPACE_BYTES",
]

EPL_OK = 0
EPL_EINVAL = -1
EPL_ERANGE = -2
EPL_ECAPACITY = -3
EPL_EHIP = -4
EPL_OUT_F32 = 0
EPL_OUT_BF16 = 1
EPL_SCALE_NONE = 0
EPL_SCALE_F32 = 1
EPL_SCALE_UE8M0 = 2
EPL_STATIC_WORKSPACE_BYTES = 8 << 20

# Every function include/epl.h declares; tests check the library exports them.
C_ENTRY_POINTS = (
    "epl_validate", "epl_workspace_bytes", "epl_capacity_rows", "epl_layout", "epl_scan",
    "epl_scatter", "epl_dispatch", "epl_scatter_fp8", "epl_dispatch_fp8", "epl_combine",
    "epl_expert_scale", "epl_status", "epl_total", "epl_strerror", "epl_version",
    "epl_ll_workspace_bytes", "epl_ll_dispatch", "epl_dispatch_static",
)


class EplError(RuntimeError):
    """A non-zero status code from libepl."""

    def __init__(self, code: int, where: str):
        self.code = code
        msg = epl_strerror(code) if _LIB is not None else f"code {code}"
        super().__init__(f"{where}: {msg} ({code})")


class Problem(ctypes.Structure):
    """epl_problem: T, K, E, R, H, S, a, G (see include/epl.h)."""

    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("scale_cols", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("ranks_per_node", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, num_tokens, num_topk, num_experts, num_ranks, hidden, scale_cols=0,
             expert_alignment=0, ranks_per_node=0):
        return cls(int(num_tokens), int(num_topk), int(num_experts), int(num_ranks), int(hidden),
                   int(scale_cols), int(expert_alignment), int(ranks_per_node), 0)

    @property
    def num_nodes(self) -> int:
        """Entries of num_tokens_per_rdma_rank (0 when it is not produced)."""
        G, R = self.ranks_per_node, self.num_ranks
        return R // G if 0 < G < R else 0

    def __repr__(self):
        return (f"Problem(T={self.num_tokens}, K={self.num_topk}, E={self.num_experts}, "
                f"R={self.num_ranks}, H={self.hidden}, S={self.scale_cols}, "
                f"a={self.expert_alignment}, G={self.ranks_per_node})")


_LIB: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_PP = ctypes.POINTER(Problem)


def lib_path() -> str:
    return _build.LIB


def is_built() -> bool:
    return os.path.exists(_build.LIB)


def ensure_built(verbose: bool = False) -> str:
    """Build libepl.so if it is missing or older than its sources."""
    if _build.needs_build():
        _build.build(verbose=verbose)
    return _build.LIB


def load() -> ctypes.CDLL:
    """Load libepl.so (or the build named by EPL_LIB, e.g. the test suite's
    host-sanitizer build); raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = os.environ.get("EPL_LIB") or _build.LIB
    if not os.path.exists(path):
        raise ImportError(
            f"libepl.so is not built ({path}); run `python -m permute_ep_layout_amd.build` "
            "or __graft_entry__.build() first. There is no fallback implementation.")
    try:
        import torch  # noqa: F401  (share torch's HIP runtime if it is loaded)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.epl_validate.argtypes = [_PP]
    lib.epl_validate.restype = i32
    lib.epl_workspace_bytes.argtypes = [_PP]
    lib.epl_workspace_bytes.restype = ctypes.c_size_t
    lib.epl_capacity_rows.argtypes = [_PP]
    lib.epl_capacity_rows.restype = i64
    lib.epl_layout.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P]
    lib.epl_layout.restype = i32
    lib.epl_scan.argtypes = [_PP, _P, _P, _P, _P, _P]
    lib.epl_scan.restype = i32
    lib.epl_scatter.argtypes = [_PP, _P, _P, _P, _P, _P, i64, _P, _P, _P, _P, _P]
    lib.epl_scatter.restype = i32
    lib.epl_dispatch.argtypes = [_PP, _P, _P, _P, i64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P]
    lib.epl_dispatch.restype = i32
    lib.epl_scatter_fp8.argtypes = [_PP, _P, _P, i32, _P, _P, _P, i64, _P, _P, _P, _P, _P]
    lib.epl_scatter_fp8.restype = i32
    lib.epl_dispatch_fp8.argtypes = [_PP, _P, _P, _P, i32, i64, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _P, _P]
    lib.epl_dispatch_fp8.restype = i32
    lib.epl_dispatch_static.argtypes = [_PP, _P, _P, _P, i64, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, ctypes.POINTER(ctypes.c_void_p), _P]
    lib.epl_dispatch_static.restype = i32
    lib.epl_ll_workspace_bytes.argtypes = [_PP, i32]
    lib.epl_ll_workspace_bytes.restype = ctypes.c_size_t
    lib.epl_ll_dispatch.argtypes = [_PP, i32, i64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.epl_ll_dispatch.restype = i32
    lib.epl_combine.argtypes = [_PP, _P, i64, _P, _P, i32, _P, _P, _P]
    lib.epl_combine.restype = i32
    lib.epl_expert_scale.argtypes = [_PP, _P, _P, i64, _P, _P, _P]
    lib.epl_expert_scale.restype = i32
    lib.epl_status.argtypes = [_P, _P]
    lib.epl_status.restype = i32
    lib.epl_total.argtypes = [_P, _P]
    lib.epl_total.restype = i64
    lib.epl_strerror.argtypes = [i32]
    lib.epl_strerror.restype = ctypes.c_char_p
    lib.epl_version.argtypes = []
    lib.epl_version.restype = i32
    _LIB = lib
    return lib


# ----------------------------------------------------------- marshalling --

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device=None) -> Optional[int]:
    if stream is None:
        torch = _torch()
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(t, name, dtype, shape=None, device=None, allow_none=False):
    torch = _torch()
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


WS_HEADER_BYTES = 256   # status word and total: all that combine / expert_scale / status touch


class StaticWorkspace:
    """The library's static workspace on one GPU (epl_dispatch_static): a
    device address, not a tensor. It can be passed wherever a workspace is
    taken after the dispatch that used it (epl_status, epl_total,
    epl_combine, epl_expert_scale)."""

    def __init__(self, address: int, device):
        self.address, self.device = int(address), device

    def data_ptr(self) -> int:
        return self.address

    def numel(self) -> int:
        return EPL_STATIC_WORKSPACE_BYTES

    def __repr__(self):
        return f"StaticWorkspace({self.address:#x}, {self.device})"


def _need_ws_arg(workspace, dev, allow_none=False):
    """A workspace argument: a uint8 tensor on `dev`, or the static workspace."""
    if isinstance(workspace, StaticWorkspace):
        if dev is not None and workspace.device != dev:
            raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
        return
    _need(workspace, "workspace", _torch().uint8, None, dev, allow_none=allow_none)


def _need_workspace(workspace, need: int, where: str):
    """The C ABI takes the workspace as a bare pointer, so its size is checked
    here, before any launch: a workspace smaller than the problem needs would
    be written past its end."""
    if need <= 0:
        raise EplError(EPL_EINVAL, where)
    if workspace.numel() < need:
        raise ValueError(f"{where}: workspace holds {workspace.numel()} bytes, the problem needs "
                         f"{need} (epl_workspace_bytes)")


def _check(rc: int, where: str):
    if rc != EPL_OK:
        raise EplError(rc, where)


def _prob(p: Problem):
    return ctypes.byref(p)


# ------------------------------------------------------- C entry points --

def epl_version() -> int:
    return load().epl_version()


def epl_strerror(code: int) -> str:
    return load().epl_strerror(int(code)).decode()


def epl_validate(p: Problem) -> int:
    return load().epl_validate(_prob(p))


def epl_workspace_bytes(p: Problem) -> int:
    return int(load().epl_workspace_bytes(_prob(p)))


def epl_capacity_rows(p: Problem) -> int:
    return int(load().epl_capacity_rows(_prob(p)))


def _need_per_node(p: Problem, t, dev):
    """num_tokens_per_rdma_rank: [R / G] int32 when the problem spans several
    nodes; otherwise None (ignored by the library)."""
    if p.num_nodes:
        _need(t, "num_tokens_per_rdma_rank", _torch().int32, (p.num_nodes,), dev)


def epl_layout(p: Problem, topk_idx, num_tokens_per_expert, num_tokens_per_rank,
               num_tokens_per_rdma_rank, is_token_in_rank, workspace, stream=None):
    torch = _torch()
    T, K, E, R = p.num_tokens, p.num_topk, p.num_experts, p.num_ranks
    _need(topk_idx, "topk_idx", torch.int64, (T, K))
    dev = topk_idx.device
    _need(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (E,), dev)
    _need(num_tokens_per_rank, "num_tokens_per_rank", torch.int32, (R,), dev)
    _need_per_node(p, num_tokens_per_rdma_rank, dev)
    _need(is_token_in_rank, "is_token_in_rank", torch.uint8, (T, R), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need_workspace(workspace, epl_workspace_bytes(p), "epl_layout")
    _check(load().epl_layout(_prob(p), _ptr(topk_idx), _ptr(num_tokens_per_expert),
                             _ptr(num_tokens_per_rank), _ptr(num_tokens_per_rdma_rank),
                             _ptr(is_token_in_rank), _ptr(workspace), _stream(stream, dev)),
           "epl_layout")


def epl_scan(p: Problem, num_tokens_per_expert, expert_start_loc, total_host, workspace,
             stream=None):
    torch = _torch()
    E = p.num_experts
    _need(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (E,))
    dev = num_tokens_per_expert.device
    _need(expert_start_loc, "expert_start_loc", torch.int32, (E,), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need_workspace(workspace, epl_workspace_bytes(p), "epl_scan")
    if total_host is not None:
        if total_host.device.type != "cpu" or not total_host.is_pinned() or \
                total_host.dtype != torch.int32 or total_host.numel() < 1:
            raise ValueError("total_host must be a pinned CPU int32 tensor")
    _check(load().epl_scan(_prob(p), _ptr(num_tokens_per_expert), _ptr(expert_start_loc),
                           _ptr(total_host), _ptr(workspace), _stream(stream, dev)), "epl_scan")


def _check_scatter_args(p, x, x_scale, topk_idx, capacity_rows, out, out_scale, m_indices,
                        output_index):
    torch = _torch()
    T, K, H, S = p.num_tokens, p.num_topk, p.hidden, p.scale_cols
    _need(topk_idx, "topk_idx", torch.int64, (T, K))
    dev = topk_idx.device
    _need(x, "x", torch.bfloat16, (T, H), dev)
    _need(out, "out", torch.bfloat16, (capacity_rows, H), dev)
    _need(m_indices, "m_indices", torch.int32, (capacity_rows,), dev)
    _need(output_index, "output_index", torch.int32, (T, K), dev)
    if S > 0:
        _need(x_scale, "x_scale", torch.float32, (T, S), dev)
        _need(out_scale, "out_scale", torch.float32, (capacity_rows, S), dev)
    elif x_scale is not None or out_scale is not None:
        raise ValueError("scale tensors given but the problem has scale_cols == 0")
    return dev


def epl_scatter(p: Problem, x, x_scale, topk_idx, expert_start_loc, workspace, capacity_rows,
                out, out_scale, m_indices, output_index, stream=None):
    torch = _torch()
    dev = _check_scatter_args(p, x, x_scale, topk_idx, capacity_rows, out, out_scale, m_indices,
                              output_index)
    _need(expert_start_loc, "expert_start_loc", torch.int32, (p.num_experts,), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need_workspace(workspace, epl_workspace_bytes(p), "epl_scatter")
    _check(load().epl_scatter(_prob(p), _ptr(x), _ptr(x_scale), _ptr(topk_idx),
                              _ptr(expert_start_loc), _ptr(workspace), int(capacity_rows),
                              _ptr(out), _ptr(out_scale), _ptr(m_indices), _ptr(output_index),
                              _stream(stream, dev)), "epl_scatter")


def epl_dispatch(p: Problem, topk_idx, x, x_scale, capacity_rows, num_tokens_per_expert,
                 num_tokens_per_rank, num_tokens_per_rdma_rank, is_token_in_rank,
                 expert_start_loc, total_host, out, out_scale, m_indices, output_index, workspace,
                 stream=None):
    torch = _torch()
    dev = _check_scatter_args(p, x, x_scale, topk_idx, capacity_rows, out, out_scale, m_indices,
                              output_index)
    E, R, T = p.num_experts, p.num_ranks, p.num_tokens
    _need(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (E,), dev)
    _need(num_tokens_per_rank, "num_tokens_per_rank", torch.int32, (R,), dev)
    _need_per_node(p, num_tokens_per_rdma_rank, dev)
    _need(is_token_in_rank, "is_token_in_rank", torch.uint8, (T, R), dev)
    _need(expert_start_loc, "expert_start_loc", torch.int32, (E,), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need_workspace(workspace, epl_workspace_bytes(p), "epl_dispatch")
    if total_host is not None and (total_host.device.type != "cpu" or not total_host.is_pinned()
                                   or total_host.dtype != torch.int32):
        raise ValueError("total_host must be a pinned CPU int32 tensor")
    _check(load().epl_dispatch(_prob(p), _ptr(topk_idx), _ptr(x), _ptr(x_scale),
                               int(capacity_rows), _ptr(num_tokens_per_expert),
                               _ptr(num_tokens_per_rank), _ptr(num_tokens_per_rdma_rank),
                               _ptr(is_token_in_rank),
                               _ptr(expert_start_loc), _ptr(total_host), _ptr(out),
                               _ptr(out_scale), _ptr(m_indices), _ptr(output_index),
                               _ptr(workspace), _stream(stream, dev)), "epl_dispatch")


def epl_dispatch_static(p: Problem, topk_idx, x, x_scale, capacity_rows, num_tokens_per_expert,
                        num_tokens_per_rank, num_tokens_per_rdma_rank, is_token_in_rank,
                        expert_start_loc, total_host, out, out_scale, m_indices, output_index,
                        stream=None) -> StaticWorkspace:
    """epl_dispatch without a workspace argument, for callers that cannot
    allocate: the library's static workspace on the current GPU is used
    (EPL_STATIC_WORKSPACE_BYTES, shared by every such call on that GPU, so
    calls that overlap on one GPU race). Returns that workspace, for
    epl_status / epl_total / epl_combine / epl_expert_scale. Problems that
    need a larger workspace are rejected."""
    torch = _torch()
    dev = _check_scatter_args(p, x, x_scale, topk_idx, capacity_rows, out, out_scale, m_indices,
                              output_index)
    E, R, T = p.num_experts, p.num_ranks, p.num_tokens
    _need(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (E,), dev)
    _need(num_tokens_per_rank, "num_tokens_per_rank", torch.int32, (R,), dev)
    _need_per_node(p, num_tokens_per_rdma_rank, dev)
    _need(is_token_in_rank, "is_token_in_rank", torch.uint8, (T, R), dev)
    _need(expert_start_loc, "expert_start_loc", torch.int32, (E,), dev)
    need = epl_workspace_bytes(p)
    if need <= 0 or need > EPL_STATIC_WORKSPACE_BYTES:
        raise ValueError(f"epl_dispatch_static: the problem needs {need} bytes of workspace, "
                         f"the static workspace holds {EPL_STATIC_WORKSPACE_BYTES}")
    if total_host is not None and (total_host.device.type != "cpu" or not total_host.is_pinned()
                                   or total_host.dtype != torch.int32):
        raise ValueError("total_host must be a pinned CPU int32 tensor")
    addr = ctypes.c_void_p()
    _check(load().epl_dispatch_static(_prob(p), _ptr(topk_idx), _ptr(x), _ptr(x_scale),
                                      int(capacity_rows), _ptr(num_tokens_per_expert),
                                      _ptr(num_tokens_per_rank), _ptr(num_tokens_per_rdma_rank),
                                      _ptr(is_token_in_rank), _ptr(expert_start_loc),
                                      _ptr(total_host), _ptr(out), _ptr(out_scale),
                                      _ptr(m_indices), _ptr(output_index), ctypes.byref(addr),
                                      _stream(stream, dev)), "epl_dispatch_static")
    return StaticWorkspace(addr.value, dev)


def _check_fp8_args(p, x, x_scale, scale_format, topk_idx, capacity_rows, out, out_scale,
                    m_indices, output_index):
    torch = _torch()
    T, K, H, S = p.num_tokens, p.num_topk, p.hidden, p.scale_cols
    _need(topk_idx, "topk_idx", torch.int64, (T, K))
    dev = topk_idx.device
    _need(x, "x", torch.uint8, (T, H), dev)
    _need(out, "out", torch.uint8, (capacity_rows, H), dev)
    _need(m_indices, "m_indices", torch.int32, (capacity_rows,), dev)
    _need(output_index, "output_index", torch.int32, (T, K), dev)
    if scale_format == EPL_SCALE_F32:
        _need(x_scale, "x_scale", torch.float32, (T, S), dev)
        _need(out_scale, "out_scale", torch.float32, (capacity_rows, S), dev)
    elif scale_format == EPL_SCALE_UE8M0:
        W = (S + 3) // 4
        _need(x_scale, "x_scale", torch.int32, (T, W), dev)
        _need(out_scale, "out_scale (column-major storage [W, capacity])", torch.int32,
              (W, capacity_rows), dev)
    elif scale_format != EPL_SCALE_NONE:
        raise ValueError(f"unknown scale format {scale_format}")
    return dev


def epl_scatter_fp8(p: Problem, x, x_scale, scale_format, topk_idx, expert_start_loc, workspace,
                    capacity_rows, out, out_scale, m_indices, output_index, stream=None):
    """FP8 rows as uint8 [T, H] (view a float8_e4m3fn tensor as uint8); the
    UE8M0 output scale buffer is int32 [W, capacity] (its transpose is the
    [capacity, W] view the grouped GEMM reads)."""
    torch = _torch()
    dev = _check_fp8_args(p, x, x_scale, scale_format, topk_idx, capacity_rows, out, out_scale,
                          m_indices, output_index)
    _need(expert_start_loc, "expert_start_loc", torch.int32, (p.num_experts,), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need_workspace(workspace, epl_workspace_bytes(p), "epl_scatter_fp8")
    _check(load().epl_scatter_fp8(_prob(p), _ptr(x), _ptr(x_scale), int(scale_format),
                                  _ptr(topk_idx), _ptr(expert_start_loc), _ptr(workspace),
                                  int(capacity_rows), _ptr(out), _ptr(out_scale), _ptr(m_indices),
                                  _ptr(output_index), _stream(stream, dev)), "epl_scatter_fp8")


def epl_dispatch_fp8(p: Problem, topk_idx, x, x_scale, scale_format, capacity_rows,
                     num_tokens_per_expert, num_tokens_per_rank, num_tokens_per_rdma_rank,
                     is_token_in_rank, expert_start_loc, total_host, out, out_scale, m_indices,
                     output_index, workspace, stream=None):
    torch = _torch()
    dev = _check_fp8_args(p, x, x_scale, scale_format, topk_idx, capacity_rows, out, out_scale,
                          m_indices, output_index)
    E, R, T = p.num_experts, p.num_ranks, p.num_tokens
    _need(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (E,), dev)
    _need(num_tokens_per_rank, "num_tokens_per_rank", torch.int32, (R,), dev)
    _need_per_node(p, num_tokens_per_rdma_rank, dev)
    _need(is_token_in_rank, "is_token_in_rank", torch.uint8, (T, R), dev)
    _need(expert_start_loc, "expert_start_loc", torch.int32, (E,), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need_workspace(workspace, epl_workspace_bytes(p), "epl_dispatch_fp8")
    if total_host is not None and (total_host.device.type != "cpu" or not total_host.is_pinned()
                                   or total_host.dtype != torch.int32):
        raise ValueError("total_host must be a pinned CPU int32 tensor")
    _check(load().epl_dispatch_fp8(_prob(p), _ptr(topk_idx), _ptr(x), _ptr(x_scale),
                                   int(scale_format), int(capacity_rows),
                                   _ptr(num_tokens_per_expert), _ptr(num_tokens_per_rank),
                                   _ptr(num_tokens_per_rdma_rank), _ptr(is_token_in_rank),
                                   _ptr(expert_start_loc),
                                   _ptr(total_host), _ptr(out), _ptr(out_scale), _ptr(m_indices),
                                   _ptr(output_index), _ptr(workspace), _stream(stream, dev)),
           "epl_dispatch_fp8")


def epl_ll_workspace_bytes(p: Problem, tokens_per_segment: int) -> int:
    return int(load().epl_ll_workspace_bytes(_prob(p), int(tokens_per_segment)))


def epl_ll_dispatch(p: Problem, tokens_per_segment, rows_per_expert, topk_idx, x, out, out_scale,
                    recv_count, src_info, layout_range, output_index, workspace, stream=None):
    """Fixed-rectangle (low-latency) dispatch; shapes as in include/epl.h:
    out uint8 [E, cap, H], out_scale f32 [E, S, cap], recv_count i32 [E],
    src_info i32 [E, cap], layout_range i32 [E, T/M, 2], output_index i32
    [T, K]; x bf16 [T, H]."""
    torch = _torch()
    T, K, E, H = p.num_tokens, p.num_topk, p.num_experts, p.hidden
    M, cap = int(tokens_per_segment), int(rows_per_expert)
    if M < 1 or T % M:
        raise ValueError("num_tokens must be a multiple of tokens_per_segment")
    _need(topk_idx, "topk_idx", torch.int64, (T, K))
    dev = topk_idx.device
    _need(x, "x", torch.bfloat16, (T, H), dev)
    _need(out, "out", torch.uint8, (E, cap, H), dev)
    _need(out_scale, "out_scale", torch.float32, (E, H // 128, cap), dev)
    _need(recv_count, "recv_count", torch.int32, (E,), dev)
    _need(src_info, "src_info", torch.int32, (E, cap), dev)
    _need(layout_range, "layout_range", torch.int32, (E, T // M, 2), dev)
    _need(output_index, "output_index", torch.int32, (T, K), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need_workspace(workspace, epl_ll_workspace_bytes(p, M), "epl_ll_dispatch")
    _check(load().epl_ll_dispatch(_prob(p), M, cap, _ptr(topk_idx), _ptr(x), _ptr(out),
                                  _ptr(out_scale), _ptr(recv_count), _ptr(src_info),
                                  _ptr(layout_range), _ptr(output_index), _ptr(workspace),
                                  _stream(stream, dev)), "epl_ll_dispatch")


def epl_combine(p: Problem, expert_out, expert_rows, output_index, topk_weights, out_dtype, y,
                workspace=None, stream=None):
    torch = _torch()
    T, K, H = p.num_tokens, p.num_topk, p.hidden
    _need(output_index, "output_index", torch.int32, (T, K))
    dev = output_index.device
    _need(expert_out, "expert_out", torch.bfloat16, (expert_rows, H), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    ydt = torch.bfloat16 if out_dtype == EPL_OUT_BF16 else torch.float32
    _need(y, "y", ydt, (T, H), dev)
    _need_ws_arg(workspace, dev, allow_none=True)
    if workspace is not None:
        _need_workspace(workspace, WS_HEADER_BYTES, "epl_combine")
    _check(load().epl_combine(_prob(p), _ptr(expert_out), int(expert_rows), _ptr(output_index),
                              _ptr(topk_weights), int(out_dtype), _ptr(y), _ptr(workspace),
                              _stream(stream, dev)), "epl_combine")


def epl_expert_scale(p: Problem, rows_in, m_indices, capacity_rows, rows_out, workspace,
                     stream=None):
    torch = _torch()
    H = p.hidden
    _need(rows_in, "rows_in", torch.bfloat16, (capacity_rows, H))
    dev = rows_in.device
    _need(m_indices, "m_indices", torch.int32, (capacity_rows,), dev)
    _need(rows_out, "rows_out", torch.bfloat16, (capacity_rows, H), dev)
    _need_ws_arg(workspace, dev)
    _need_workspace(workspace, WS_HEADER_BYTES, "epl_expert_scale")
    _check(load().epl_expert_scale(_prob(p), _ptr(rows_in), _ptr(m_indices), int(capacity_rows),
                                   _ptr(rows_out), _ptr(workspace), _stream(stream, dev)),
           "epl_expert_scale")


def epl_status(workspace, stream=None) -> int:
    _need_workspace(workspace, WS_HEADER_BYTES, "epl_status")
    return int(load().epl_status(_ptr(workspace), _stream(stream, workspace.device)))


def epl_total(workspace, stream=None) -> int:
    _need_workspace(workspace, WS_HEADER_BYTES, "epl_total")
    n = int(load().epl_total(_ptr(workspace), _stream(stream, workspace.device)))
    if n < 0:
        raise EplError(n, "epl_total")
    return n


def prepare(name: str, *args, stream=None):
    """A zero-overhead caller of C entry point `name` with fixed arguments:
    tensors become their device addresses, a Problem is passed by reference,
    and the stream (default: torch's current stream) is resolved once. The
    arguments are not checked here: call the checked ``epl_*`` wrapper with
    the same arguments first (e.g. in a warm-up). Raises EplError on a non-zero
    return code."""
    import torch
    fn = getattr(load(), name)
    cargs = []
    for a in args:
        if isinstance(a, Problem):
            cargs.append(ctypes.byref(a))
        elif isinstance(a, torch.Tensor):
            cargs.append(ctypes.c_void_p(a.data_ptr()))
        else:
            cargs.append(a)
    cargs.append(ctypes.c_void_p(_stream(stream)))

    def call():
        rc = fn(*cargs)
        if rc != EPL_OK:
            raise EplError(rc, name)
    return call


# ------------------------------------------------------- tensor helpers --

class DispatchResult(NamedTuple):
    out: "torch.Tensor"                  # [capacity, H] bf16 (rows >= total unwritten)
    out_scale: Optional["torch.Tensor"]  # [capacity, S] f32 or None
    m_indices: "torch.Tensor"            # [capacity] i32
    output_index: "torch.Tensor"         # [T, K] i32
    expert_start_loc: "torch.Tensor"     # [E] i32
    num_tokens_per_expert: "torch.Tensor"
    num_tokens_per_rank: "torch.Tensor"
    num_tokens_per_rdma_rank: Optional["torch.Tensor"]   # [R / G] i32, None on one node
    is_token_in_rank: "torch.Tensor"     # [T, R] u8 (0/1)
    total_host: "torch.Tensor"           # pinned [1] i32, valid after the stream syncs
    workspace: "torch.Tensor"
    problem: Problem

    def total(self) -> int:
        """Routed row count N (synchronises the current stream)."""
        _torch().cuda.current_stream(self.out.device).synchronize()
        return int(self.total_host[0])


def workspace_for(p: Problem, device):
    torch = _torch()
    n = epl_workspace_bytes(p)
    if n == 0:
        raise EplError(EPL_EINVAL, "epl_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dispatch(x, topk_idx, num_experts: int, num_ranks: int, x_scale=None,
             capacity: Optional[int] = None, mode: str = "capacity", workspace=None,
             stream=None, expert_alignment: int = 0, ranks_per_node: int = 0) -> DispatchResult:
    """Layout + scan + scatter.

    mode="capacity" (default): one epl_dispatch call; the output buffers have
    `capacity` rows (default epl_capacity_rows, which always suffices) and no
    host wait happens. mode="exact": epl_layout + epl_scan, then the host waits for the
    total N, allocates exactly N rows and calls epl_scatter.

    Receive side: pass the rank's local expert ids (-1 for other ranks'
    experts) with num_experts = the local expert count and num_ranks = 1.
    """
    torch = _torch()
    T, H = x.shape
    K = topk_idx.shape[1]
    S = 0 if x_scale is None else x_scale.shape[1]
    p = Problem.make(T, K, num_experts, num_ranks, H, S, expert_alignment, ranks_per_node)
    _check(epl_validate(p), "epl_validate")
    dev = x.device
    ws = workspace if workspace is not None else workspace_for(p, dev)
    i32 = torch.int32
    cnt = torch.empty(num_experts, dtype=i32, device=dev)
    per_rank = torch.empty(num_ranks, dtype=i32, device=dev)
    per_node = torch.empty(p.num_nodes, dtype=i32, device=dev) if p.num_nodes else None
    in_rank = torch.empty((T, num_ranks), dtype=torch.uint8, device=dev)
    start = torch.empty(num_experts, dtype=i32, device=dev)
    oi = torch.empty((T, K), dtype=i32, device=dev)
    total_host = torch.zeros(1, dtype=i32, pin_memory=True)
    if mode == "capacity":
        cap = epl_capacity_rows(p) if capacity is None else int(capacity)
        out = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        out_scale = torch.empty((cap, S), dtype=torch.float32, device=dev) if S else None
        m_idx = torch.empty(cap, dtype=i32, device=dev)
        epl_dispatch(p, topk_idx, x, x_scale, cap, cnt, per_rank, per_node, in_rank, start,
                     total_host, out, out_scale, m_idx, oi, ws, stream)
    elif mode == "exact":
        epl_layout(p, topk_idx, cnt, per_rank, per_node, in_rank, ws, stream)
        epl_scan(p, cnt, start, total_host, ws, stream)
        torch.cuda.current_stream(dev).synchronize() if stream is None else stream.synchronize()
        cap = int(total_host[0])
        out = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        out_scale = torch.empty((cap, S), dtype=torch.float32, device=dev) if S else None
        m_idx = torch.empty(cap, dtype=i32, device=dev)
        epl_scatter(p, x, x_scale, topk_idx, start, ws, cap, out, out_scale, m_idx, oi, stream)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return DispatchResult(out, out_scale, m_idx, oi, start, cnt, per_rank, per_node, in_rank,
                          total_host, ws, p)


def combine(expert_out, output_index, topk_weights, out_dtype=None, workspace=None,
            stream=None):
    """y[t] = sum_k w[t,k] * expert_out[output_index[t,k]] (fp32 accumulation)."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    T, K = output_index.shape
    rows, H = expert_out.shape
    p = Problem.make(T, K, 1, 1, H, 0)
    code = EPL_OUT_BF16 if out_dtype == torch.bfloat16 else EPL_OUT_F32
    y = torch.empty((T, H), dtype=out_dtype, device=expert_out.device)
    epl_combine(p, expert_out, rows, output_index, topk_weights, code, y, workspace, stream)
    return y


def expert_scale(res: DispatchResult, rows_in=None, stream=None):
    """The large-batch workload's synthetic expert applied to a dispatch result."""
    torch = _torch()
    rows_in = res.out if rows_in is None else rows_in
    out = torch.empty_like(rows_in)
    epl_expert_scale(res.problem, rows_in, res.m_indices, rows_in.shape[0], out, res.workspace,
                     stream)
    return out
