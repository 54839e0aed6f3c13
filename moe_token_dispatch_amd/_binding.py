"""ctypes binding of the dispatch C ABI (``include/moe_dispatch.h``).

Argument marshalling only: every step of dispatch runs in the HIP kernels of
``libmoe_dispatch.so``. torch supplies device memory and the current stream.
The library must have been built (``python -m moe_token_dispatch_amd.build``);
loading fails loudly otherwise, and there is no fallback path.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch  # load torch's HIP runtime first so the library binds to the same one

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_dispatch.so")

ABI_VERSION = 6
MAX_TOPK = 32
MAX_EXPERTS = 4096
MAX_RANKS = 1024

OK = 0
ERR_NULL = -1
ERR_ARG = -2
ERR_ALIGN = -3
ERR_WORKSPACE = -4
ERR_HIP = -5

STATUS_BAD_EXPERT = 1
STATUS_RECV_OVERFLOW = 2
STATUS_RANK_OVERFLOW = 4
STATUS_DUP_EXPERT = 8
STATUS_BAD_COUNT = 16
STATUS_TIMEOUT = 32
DEFAULT_WAIT_LIMIT = 1 << 20

RANK_CONTIG = 1
EXPERT_MAJOR = 2
ZERO_PAD = 4
ALL_OUTPUTS = RANK_CONTIG | EXPERT_MAJOR | ZERO_PAD
ROWS_READ_AHEAD = 8  # scatter hint: the rows were just read ahead (changes no result)


class DispatchError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {dispatch_strerror(code)} (code {code})")


class Problem(ctypes.Structure):
    """dispatch_problem_t."""

    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("topk_idx_bytes", ctypes.c_int32),
        ("sf_per_token", ctypes.c_int32),
        ("row_bytes", ctypes.c_int64),
        ("recv_capacity_rows", ctypes.c_int64),
        ("rank_capacity_rows", ctypes.c_int64),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class LayoutPtrs(ctypes.Structure):
    """dispatch_layout_t."""

    _fields_ = [(name, ctypes.c_void_p) for name in (
        "expert_count", "rank_count", "expert_psum", "rank_psum", "expert_slot", "rank_slot",
        "recv_src_token_idx", "rank_src_token_idx", "status", "expert_count_cumulative")]


class ExpandProblem(ctypes.Structure):
    """dispatch_expand_problem_t."""

    _fields_ = [
        ("num_sources", ctypes.c_int32),
        ("rows_per_source", ctypes.c_int32),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("local_rank", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("topk_idx_bytes", ctypes.c_int32),
        ("sf_per_token", ctypes.c_int32),
        ("reserved", ctypes.c_uint32),
        ("row_bytes", ctypes.c_int64),
        ("recv_capacity_rows", ctypes.c_int64),
    ]


class CombineProblem(ctypes.Structure):
    """dispatch_combine_problem_t."""

    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("num_topk", ctypes.c_int32),
        ("reserved", ctypes.c_uint32),
        ("hidden", ctypes.c_int64),
        ("expert_rows", ctypes.c_int64),
    ]


_LIB = None

# Exported symbols of include/moe_dispatch.h.
SYMBOLS = ("dispatch_abi_version", "dispatch_strerror", "dispatch_workspace_size",
           "dispatch_max_rows", "dispatch_layout", "dispatch_layout_read_ahead",
           "dispatch_scatter", "dispatch_layout_and_scatter", "dispatch_layout_and_scatter_noalloc",
           "dispatch_kernel_count", "dispatch_set_wait_limit",
           "dispatch_expand_workspace_size", "dispatch_expand_max_rows", "dispatch_expand_layout",
           "dispatch_expand_scatter", "dispatch_expand_layout_and_scatter", "dispatch_combine")


def load_library(path: str = LIB_PATH):
    """Load libmoe_dispatch.so (built in-tree) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m moe_token_dispatch_amd.build`")
    lib = ctypes.CDLL(path)
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.dispatch_abi_version.argtypes = []
    lib.dispatch_abi_version.restype = i
    lib.dispatch_strerror.argtypes = [i]
    lib.dispatch_strerror.restype = ctypes.c_char_p
    lib.dispatch_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(sz)]
    lib.dispatch_workspace_size.restype = i
    lib.dispatch_max_rows.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_int64)]
    lib.dispatch_max_rows.restype = i
    lib.dispatch_layout.argtypes = [ctypes.POINTER(Problem), p, ctypes.POINTER(LayoutPtrs), p, sz, p]
    lib.dispatch_layout.restype = i
    lib.dispatch_layout_read_ahead.argtypes = [ctypes.POINTER(Problem), p, ctypes.POINTER(LayoutPtrs), p, sz, p, p,
                                               p]
    lib.dispatch_layout_read_ahead.restype = i
    lib.dispatch_scatter.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(LayoutPtrs), p, p, p, p, p, p, p]
    lib.dispatch_scatter.restype = i
    lib.dispatch_layout_and_scatter.argtypes = [ctypes.POINTER(Problem), p, ctypes.POINTER(LayoutPtrs), p, sz,
                                                p, p, p, p, p, p, p]
    lib.dispatch_layout_and_scatter.restype = i
    lib.dispatch_layout_and_scatter_noalloc.argtypes = [ctypes.POINTER(Problem), p, ctypes.POINTER(LayoutPtrs),
                                                        p, p, p, p, p, p, p]
    lib.dispatch_layout_and_scatter_noalloc.restype = i
    lib.dispatch_kernel_count.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.dispatch_kernel_count.restype = i
    lib.dispatch_set_wait_limit.argtypes = [ctypes.c_int64]
    lib.dispatch_set_wait_limit.restype = i
    ep = ctypes.POINTER(ExpandProblem)
    lib.dispatch_expand_workspace_size.argtypes = [ep, ctypes.POINTER(sz)]
    lib.dispatch_expand_workspace_size.restype = i
    lib.dispatch_expand_max_rows.argtypes = [ep, ctypes.POINTER(ctypes.c_int64)]
    lib.dispatch_expand_max_rows.restype = i
    lib.dispatch_expand_layout.argtypes = [ep, p, p, ctypes.POINTER(LayoutPtrs), p, sz, p]
    lib.dispatch_expand_layout.restype = i
    lib.dispatch_expand_scatter.argtypes = [ep, ctypes.POINTER(LayoutPtrs), p, p, p, p, p]
    lib.dispatch_expand_layout_and_scatter.argtypes = [ep, p, p, ctypes.POINTER(LayoutPtrs), p, sz, p, p, p, p, p]
    lib.dispatch_expand_layout_and_scatter.restype = i
    lib.dispatch_expand_scatter.restype = i
    lib.dispatch_combine.argtypes = [ctypes.POINTER(CombineProblem), p, p, p, p, p]
    lib.dispatch_combine.restype = i
    if lib.dispatch_abi_version() != ABI_VERSION:
        raise ImportError(f"{path}: ABI version {lib.dispatch_abi_version()} != {ABI_VERSION}")
    _LIB = lib
    return lib


# ---------------------------------------------------------------- C ABI calls


def dispatch_abi_version() -> int:
    return load_library().dispatch_abi_version()


def dispatch_strerror(code: int) -> str:
    return load_library().dispatch_strerror(code).decode()


def dispatch_workspace_size(problem: Problem) -> int:
    out = ctypes.c_size_t(0)
    rc = load_library().dispatch_workspace_size(ctypes.byref(problem), ctypes.byref(out))
    if rc:
        raise DispatchError(rc, "dispatch_workspace_size")
    return int(out.value)


def dispatch_max_rows(problem: Problem) -> Tuple[int, int]:
    recv, rank = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = load_library().dispatch_max_rows(ctypes.byref(problem), ctypes.byref(recv), ctypes.byref(rank))
    if rc:
        raise DispatchError(rc, "dispatch_max_rows")
    return int(recv.value), int(rank.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream: Optional[torch.cuda.Stream], device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


@dataclasses.dataclass
class LayoutTensors:
    """Device int32 outputs of dispatch_layout (see dispatch_layout_t)."""

    expert_count: torch.Tensor
    rank_count: torch.Tensor
    expert_psum: torch.Tensor
    rank_psum: torch.Tensor
    expert_slot: torch.Tensor
    rank_slot: torch.Tensor
    recv_src_token_idx: torch.Tensor
    rank_src_token_idx: torch.Tensor
    status: torch.Tensor

    def ptrs(self, expert_count_cumulative: Optional[torch.Tensor] = None) -> LayoutPtrs:
        return LayoutPtrs(*[t.data_ptr() for t in (
            self.expert_count, self.rank_count, self.expert_psum, self.rank_psum, self.expert_slot,
            self.rank_slot, self.recv_src_token_idx, self.rank_src_token_idx, self.status)],
            _ptr(expert_count_cumulative))

    def tensors(self):
        """(name, tensor) of every output present."""
        return [(f.name, getattr(self, f.name)) for f in dataclasses.fields(self) if getattr(self, f.name) is not None]


def _fields_of(layout):
    """(name, tensor) of every layout output present (optional ones may be None)."""
    return [(f.name, getattr(layout, f.name)) for f in dataclasses.fields(layout) if getattr(layout, f.name) is not None]


def _check_device_tensor(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _check_cumulative(t: Optional[torch.Tensor], num_experts: int) -> None:
    if t is not None:
        _check_device_tensor(t, "expert_count_cumulative", torch.int32)
        if t.numel() < num_experts:
            raise ValueError(f"expert_count_cumulative needs {num_experts} entries, has {t.numel()}")


# The C ABI takes raw pointers and trusts their sizes; the binding knows every
# size from the problem and refuses a tensor too small for it, before any call.
def _need(t: Optional[torch.Tensor], name: str, nbytes: int) -> None:
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes; the problem needs {nbytes}")


def _check_dispatch_sizes(problem: Problem, topk_idx: Optional[torch.Tensor], layout: "LayoutTensors") -> None:
    t, k, e, r = problem.num_tokens, problem.num_topk, problem.num_experts, problem.num_ranks
    _need(topk_idx, "topk_idx", t * k * problem.topk_idx_bytes)
    for name, n in (("expert_count", e), ("rank_count", r), ("expert_psum", e + 1), ("rank_psum", r + 1),
                    ("expert_slot", t * k), ("rank_slot", t * k),
                    ("recv_src_token_idx", problem.recv_capacity_rows),
                    ("rank_src_token_idx", problem.rank_capacity_rows), ("status", 1)):
        _need(getattr(layout, name), name, 4 * n)


def _check_dispatch_rows(problem: Problem, x, x_sf, rank_x, rank_sf, recv_x, recv_sf) -> None:
    t, rb, s = problem.num_tokens, problem.row_bytes, problem.sf_per_token
    _need(x, "x", t * rb)
    _need(x_sf, "x_sf", 4 * t * s)
    if problem.flags & RANK_CONTIG:
        _need(rank_x, "rank_x", problem.rank_capacity_rows * rb)
        _need(rank_sf, "rank_sf", 4 * problem.rank_capacity_rows * s)
    if problem.flags & EXPERT_MAJOR:
        _need(recv_x, "recv_x", problem.recv_capacity_rows * rb)
        _need(recv_sf, "recv_sf", 4 * problem.recv_capacity_rows * s)


def _check_expand_sizes(problem: "ExpandProblem", recv_topk_idx, recv_count, layout, recv_buf, recv_sf_buf,
                        recv_x, recv_sf) -> None:
    rows = problem.num_sources * problem.rows_per_source
    local = problem.num_experts // problem.num_ranks
    cap, rb, s = problem.recv_capacity_rows, problem.row_bytes, problem.sf_per_token
    _need(recv_topk_idx, "recv_topk_idx", rows * problem.num_topk * problem.topk_idx_bytes)
    _need(recv_count, "recv_count", 4 * problem.num_sources)
    if layout is not None:
        for name, n in (("expert_count", local), ("expert_psum", local + 1), ("expert_slot", rows * problem.num_topk),
                        ("recv_src_row_idx", cap), ("status", 1)):
            _need(getattr(layout, name), name, 4 * n)
    _need(recv_buf, "recv_buf", rows * rb)
    _need(recv_sf_buf, "recv_sf_buf", 4 * rows * s)
    _need(recv_x, "recv_x", cap * rb)
    _need(recv_sf, "recv_sf", 4 * cap * s)


def dispatch_layout(problem: Problem, topk_idx: torch.Tensor, out: LayoutTensors,
                    workspace: torch.Tensor, stream: Optional[torch.cuda.Stream] = None,
                    expert_count_cumulative: Optional[torch.Tensor] = None) -> None:
    """Enqueue Count -> Prefix Sum -> slot assignment on the stream. When
    ``expert_count_cumulative`` (device int32 [E], kept by the caller) is given,
    a successful call adds its expert_count to it."""
    _check_device_tensor(topk_idx, "topk_idx")
    if topk_idx.element_size() != problem.topk_idx_bytes:
        raise ValueError("topk_idx element width does not match problem.topk_idx_bytes")
    _check_device_tensor(workspace, "workspace")
    for name, t in _fields_of(out):
        _check_device_tensor(t, name, torch.int32)
    _check_cumulative(expert_count_cumulative, problem.num_experts)
    _check_dispatch_sizes(problem, topk_idx, out)
    lay = out.ptrs(expert_count_cumulative)
    rc = load_library().dispatch_layout(ctypes.byref(problem), _ptr(topk_idx), ctypes.byref(lay),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream_handle(stream, topk_idx.device))
    if rc:
        raise DispatchError(rc, "dispatch_layout")


def dispatch_layout_read_ahead(problem: Problem, topk_idx: torch.Tensor, out: LayoutTensors,
                               workspace: torch.Tensor, x: torch.Tensor, x_sf: Optional[torch.Tensor] = None,
                               stream: Optional[torch.cuda.Stream] = None,
                               expert_count_cumulative: Optional[torch.Tensor] = None) -> None:
    """dispatch_layout, reading the token rows ``x`` (and ``x_sf``) into the
    Infinity Cache while it runs, for a dispatch_scatter of them that follows."""
    _check_device_tensor(topk_idx, "topk_idx")
    if topk_idx.element_size() != problem.topk_idx_bytes:
        raise ValueError("topk_idx element width does not match problem.topk_idx_bytes")
    _check_device_tensor(workspace, "workspace")
    _check_device_tensor(x, "x")
    if x_sf is not None:
        _check_device_tensor(x_sf, "x_sf")
    for name, t in _fields_of(out):
        _check_device_tensor(t, name, torch.int32)
    _check_cumulative(expert_count_cumulative, problem.num_experts)
    _check_dispatch_sizes(problem, topk_idx, out)
    _need(x, "x", problem.num_tokens * problem.row_bytes)
    _need(x_sf, "x_sf", 4 * problem.num_tokens * problem.sf_per_token)
    lay = out.ptrs(expert_count_cumulative)
    rc = load_library().dispatch_layout_read_ahead(ctypes.byref(problem), _ptr(topk_idx), ctypes.byref(lay),
                                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _ptr(x), _ptr(x_sf), _stream_handle(stream, topk_idx.device))
    if rc:
        raise DispatchError(rc, "dispatch_layout_read_ahead")


def dispatch_scatter(problem: Problem, layout: LayoutTensors, x: torch.Tensor,
                     x_sf: Optional[torch.Tensor], rank_x: Optional[torch.Tensor],
                     rank_sf: Optional[torch.Tensor], recv_x: Optional[torch.Tensor],
                     recv_sf: Optional[torch.Tensor], stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueue the row scatter of a layout on the stream."""
    _check_device_tensor(x, "x")
    for name, t in (("x_sf", x_sf), ("rank_x", rank_x), ("rank_sf", rank_sf), ("recv_x", recv_x),
                    ("recv_sf", recv_sf)):
        if t is not None:
            _check_device_tensor(t, name)
    for name, t in _fields_of(layout):
        _check_device_tensor(t, name, torch.int32)
    _check_dispatch_sizes(problem, None, layout)
    _check_dispatch_rows(problem, x, x_sf, rank_x, rank_sf, recv_x, recv_sf)
    lay = layout.ptrs()
    rc = load_library().dispatch_scatter(ctypes.byref(problem), ctypes.byref(lay), _ptr(x), _ptr(x_sf),
                                         _ptr(rank_x), _ptr(rank_sf), _ptr(recv_x), _ptr(recv_sf),
                                         _stream_handle(stream, x.device))
    if rc:
        raise DispatchError(rc, "dispatch_scatter")


def dispatch_kernel_count(problem: Problem) -> tuple:
    """(kernels of dispatch_layout, kernels of dispatch_layout_and_scatter) for this problem."""
    lay, both = ctypes.c_int(0), ctypes.c_int(0)
    rc = load_library().dispatch_kernel_count(ctypes.byref(problem), ctypes.byref(lay), ctypes.byref(both))
    if rc:
        raise DispatchError(rc, "dispatch_kernel_count")
    return lay.value, both.value


def dispatch_set_wait_limit(polls: int) -> None:
    """Bound the one-launch layout's in-kernel wait to `polls` polls (0: the default); process-wide."""
    rc = load_library().dispatch_set_wait_limit(int(polls))
    if rc:
        raise DispatchError(rc, "dispatch_set_wait_limit")


def dispatch_layout_and_scatter(problem: Problem, topk_idx: torch.Tensor, out: LayoutTensors,
                                workspace: torch.Tensor, x: torch.Tensor, x_sf: Optional[torch.Tensor],
                                rank_x: Optional[torch.Tensor], rank_sf: Optional[torch.Tensor],
                                recv_x: Optional[torch.Tensor], recv_sf: Optional[torch.Tensor],
                                stream: Optional[torch.cuda.Stream] = None,
                                expert_count_cumulative: Optional[torch.Tensor] = None) -> None:
    """Enqueue dispatch_layout then dispatch_scatter as one call (one kernel
    for a batch that fits one layout tile)."""
    _check_device_tensor(topk_idx, "topk_idx")
    if topk_idx.element_size() != problem.topk_idx_bytes:
        raise ValueError("topk_idx element width does not match problem.topk_idx_bytes")
    _check_device_tensor(workspace, "workspace")
    for name, t in _fields_of(out):
        _check_device_tensor(t, name, torch.int32)
    _check_cumulative(expert_count_cumulative, problem.num_experts)
    _check_device_tensor(x, "x")
    for name, t in (("x_sf", x_sf), ("rank_x", rank_x), ("rank_sf", rank_sf), ("recv_x", recv_x),
                    ("recv_sf", recv_sf)):
        if t is not None:
            _check_device_tensor(t, name)
    _check_dispatch_sizes(problem, topk_idx, out)
    _check_dispatch_rows(problem, x, x_sf, rank_x, rank_sf, recv_x, recv_sf)
    lay = out.ptrs(expert_count_cumulative)
    rc = load_library().dispatch_layout_and_scatter(
        ctypes.byref(problem), _ptr(topk_idx), ctypes.byref(lay), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(x), _ptr(x_sf), _ptr(rank_x), _ptr(rank_sf),
        _ptr(recv_x), _ptr(recv_sf), _stream_handle(stream, topk_idx.device))
    if rc:
        raise DispatchError(rc, "dispatch_layout_and_scatter")


def dispatch_layout_and_scatter_noalloc(problem: Problem, topk_idx: torch.Tensor, out: LayoutTensors,
                                        x: torch.Tensor, x_sf: Optional[torch.Tensor],
                                        rank_x: Optional[torch.Tensor], rank_sf: Optional[torch.Tensor],
                                        recv_x: Optional[torch.Tensor], recv_sf: Optional[torch.Tensor],
                                        stream: Optional[torch.cuda.Stream] = None,
                                        expert_count_cumulative: Optional[torch.Tensor] = None) -> None:
    """dispatch_layout_and_scatter with the library's own fixed workspace (no
    workspace argument, nothing allocated). Calls that overlap on one GPU race."""
    _check_device_tensor(topk_idx, "topk_idx")
    if topk_idx.element_size() != problem.topk_idx_bytes:
        raise ValueError("topk_idx element width does not match problem.topk_idx_bytes")
    for name, t in _fields_of(out):
        _check_device_tensor(t, name, torch.int32)
    _check_cumulative(expert_count_cumulative, problem.num_experts)
    _check_device_tensor(x, "x")
    for name, t in (("x_sf", x_sf), ("rank_x", rank_x), ("rank_sf", rank_sf), ("recv_x", recv_x),
                    ("recv_sf", recv_sf)):
        if t is not None:
            _check_device_tensor(t, name)
    _check_dispatch_sizes(problem, topk_idx, out)
    _check_dispatch_rows(problem, x, x_sf, rank_x, rank_sf, recv_x, recv_sf)
    lay = out.ptrs(expert_count_cumulative)
    rc = load_library().dispatch_layout_and_scatter_noalloc(
        ctypes.byref(problem), _ptr(topk_idx), ctypes.byref(lay), _ptr(x), _ptr(x_sf), _ptr(rank_x),
        _ptr(rank_sf), _ptr(recv_x), _ptr(recv_sf), _stream_handle(stream, topk_idx.device))
    if rc:
        raise DispatchError(rc, "dispatch_layout_and_scatter_noalloc")


# ------------------------------------------------- allocation helpers (plumbing)


def make_problem(num_tokens: int, num_topk: int, num_experts: int, num_ranks: int,
                 expert_alignment: int = 1, topk_idx_bytes: int = 8, row_bytes: int = 0,
                 sf_per_token: int = 0, recv_capacity_rows: Optional[int] = None,
                 rank_capacity_rows: Optional[int] = None, flags: int = ALL_OUTPUTS) -> Problem:
    """A problem; capacities default to the library's worst-case row counts."""
    p = Problem(num_tokens, num_topk, num_experts, num_ranks, expert_alignment, topk_idx_bytes,
                sf_per_token, row_bytes, 0, 0, flags, 0)
    max_recv, max_rank = dispatch_max_rows(p)
    p.recv_capacity_rows = max_recv if recv_capacity_rows is None else recv_capacity_rows
    p.rank_capacity_rows = max_rank if rank_capacity_rows is None else rank_capacity_rows
    return p


def alloc_layout(problem: Problem, device) -> LayoutTensors:
    i32 = dict(dtype=torch.int32, device=device)
    t, k = problem.num_tokens, problem.num_topk
    return LayoutTensors(
        expert_count=torch.empty(problem.num_experts, **i32),
        rank_count=torch.empty(problem.num_ranks, **i32),
        expert_psum=torch.empty(problem.num_experts + 1, **i32),
        rank_psum=torch.empty(problem.num_ranks + 1, **i32),
        expert_slot=torch.empty((t, k), **i32),
        rank_slot=torch.empty((t, k), **i32),
        recv_src_token_idx=torch.empty(max(problem.recv_capacity_rows, 1), **i32),
        rank_src_token_idx=torch.empty(max(problem.rank_capacity_rows, 1), **i32),
        status=torch.empty(1, **i32))


def alloc_workspace(problem: Problem, device) -> torch.Tensor:
    """Workspace for the layout calls: zero-filled, as its first use requires (torch allocations are
    256-byte aligned)."""
    n = dispatch_workspace_size(problem)
    return torch.zeros((n + 255) // 256 * 256, dtype=torch.uint8, device=device)


@dataclasses.dataclass
class RowBuffers:
    rank_x: Optional[torch.Tensor]   # uint8 [rank_capacity_rows, row_bytes]
    rank_sf: Optional[torch.Tensor]  # float32 [rank_capacity_rows, S]
    recv_x: Optional[torch.Tensor]   # uint8 [recv_capacity_rows, row_bytes]
    recv_sf: Optional[torch.Tensor]  # float32 [recv_capacity_rows, S]


def alloc_rows(problem: Problem, device) -> RowBuffers:
    rb, s = problem.row_bytes, problem.sf_per_token
    want_rank = bool(problem.flags & RANK_CONTIG)
    want_expert = bool(problem.flags & EXPERT_MAJOR)

    def rows(n, width, dtype, on):
        return torch.empty((max(n, 1), width), dtype=dtype, device=device) if on and width > 0 else None

    return RowBuffers(rank_x=rows(problem.rank_capacity_rows, rb, torch.uint8, want_rank),
                      rank_sf=rows(problem.rank_capacity_rows, s, torch.float32, want_rank),
                      recv_x=rows(problem.recv_capacity_rows, rb, torch.uint8, want_expert),
                      recv_sf=rows(problem.recv_capacity_rows, s, torch.float32, want_expert))


class Plan:
    """A prepared dispatch: the problem, the tensors and the stream are checked
    once and the C arguments are built once, so each call is a single C call.

    ``layout()`` enqueues dispatch_layout, ``scatter()`` enqueues
    dispatch_scatter, ``__call__`` enqueues both as one
    dispatch_layout_and_scatter call; ``layout_read_ahead()`` followed by
    ``scatter(read_ahead=True)`` is that call's two halves. The tensors must stay alive and keep
    their storage while the plan is used.
    """

    def __init__(self, problem: Problem, topk_idx: torch.Tensor, layout: LayoutTensors,
                 workspace: torch.Tensor, x: Optional[torch.Tensor] = None,
                 x_sf: Optional[torch.Tensor] = None, rows: Optional[RowBuffers] = None,
                 stream: Optional[torch.cuda.Stream] = None,
                 expert_count_cumulative: Optional[torch.Tensor] = None):
        _check_device_tensor(topk_idx, "topk_idx")
        if topk_idx.element_size() != problem.topk_idx_bytes:
            raise ValueError("topk_idx element width does not match problem.topk_idx_bytes")
        _check_device_tensor(workspace, "workspace")
        for name, t in _fields_of(layout):
            _check_device_tensor(t, name, torch.int32)
        _check_cumulative(expert_count_cumulative, problem.num_experts)
        _check_dispatch_sizes(problem, topk_idx, layout)
        # The plan keeps its own copy of the problem: the tensor sizes were
        # checked against these values, and a later change to the caller's
        # struct must not reach the C calls.
        problem = Problem.from_buffer_copy(problem)
        self._problem = problem
        self._lib = load_library()
        self._keep = (problem, topk_idx, layout, workspace, x, x_sf, rows, expert_count_cumulative)
        self._lay = layout.ptrs(expert_count_cumulative)
        handle = _stream_handle(stream, topk_idx.device)
        self._layout_args = (ctypes.byref(problem), _ptr(topk_idx), ctypes.byref(self._lay), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), handle)
        self._scatter_args = self._scatter_ra_args = self._both_args = self._layout_ra_args = None
        if x is not None:
            _check_device_tensor(x, "x")
            rows = rows if rows is not None else RowBuffers(None, None, None, None)
            for name in ("rank_x", "rank_sf", "recv_x", "recv_sf"):
                t = getattr(rows, name)
                if t is not None:
                    _check_device_tensor(t, name)
            if x_sf is not None:
                _check_device_tensor(x_sf, "x_sf")
            _check_dispatch_rows(problem, x, x_sf, rows.rank_x, rows.rank_sf, rows.recv_x, rows.recv_sf)
            row_ptrs = (_ptr(x), _ptr(x_sf), _ptr(rows.rank_x), _ptr(rows.rank_sf), _ptr(rows.recv_x),
                        _ptr(rows.recv_sf))
            self._scatter_args = (ctypes.byref(problem), ctypes.byref(self._lay), *row_ptrs, handle)
            # The same problem with the read-ahead hint, for the scatter that
            # follows layout_read_ahead().
            ra_problem = Problem.from_buffer_copy(problem)
            ra_problem.flags |= ROWS_READ_AHEAD
            self._keep += (ra_problem,)
            self._scatter_ra_args = (ctypes.byref(ra_problem), *self._scatter_args[1:])
            self._both_args = (*self._layout_args[:-1], *row_ptrs, handle)
            self._layout_ra_args = (*self._layout_args[:-1], _ptr(x), _ptr(x_sf), handle)

    def layout(self) -> None:
        rc = self._lib.dispatch_layout(*self._layout_args)
        if rc:
            raise DispatchError(rc, "dispatch_layout")

    def layout_read_ahead(self) -> None:
        """dispatch_layout_read_ahead: the layout, reading the plan's token rows
        into the Infinity Cache for the scatter that follows."""
        if self._layout_ra_args is None:
            raise ValueError("this plan has no token batch to read ahead")
        rc = self._lib.dispatch_layout_read_ahead(*self._layout_ra_args)
        if rc:
            raise DispatchError(rc, "dispatch_layout_read_ahead")

    def scatter(self, read_ahead: bool = False) -> None:
        """dispatch_scatter; ``read_ahead``: right after layout_read_ahead()
        (sets DISPATCH_ROWS_READ_AHEAD)."""
        if self._scatter_args is None:
            raise ValueError("this plan has no token batch to scatter")
        rc = self._lib.dispatch_scatter(*(self._scatter_ra_args if read_ahead else self._scatter_args))
        if rc:
            raise DispatchError(rc, "dispatch_scatter")

    def __call__(self) -> None:
        if self._scatter_args is None:
            raise ValueError("this plan has no token batch to scatter")
        rc = self._lib.dispatch_layout_and_scatter(*self._both_args)
        if rc:
            raise DispatchError(rc, "dispatch_layout_and_scatter")


# ------------------------------------------------------------ receiver-side expand


def make_expand_problem(num_sources: int, rows_per_source: int, num_topk: int, num_experts: int,
                        num_ranks: int, local_rank: int, expert_alignment: int = 1, topk_idx_bytes: int = 8,
                        row_bytes: int = 16, sf_per_token: int = 0,
                        recv_capacity_rows: Optional[int] = None) -> ExpandProblem:
    """An expand problem; the capacity defaults to the library's worst case."""
    q = ExpandProblem(num_sources, rows_per_source, num_topk, num_experts, num_ranks, local_rank,
                      expert_alignment, topk_idx_bytes, sf_per_token, 0, row_bytes, 0)
    cap = ctypes.c_int64(0)
    rc = load_library().dispatch_expand_max_rows(ctypes.byref(q), ctypes.byref(cap))
    if rc:
        raise DispatchError(rc, "dispatch_expand_max_rows")
    q.recv_capacity_rows = int(cap.value) if recv_capacity_rows is None else recv_capacity_rows
    return q


def dispatch_expand_workspace_size(problem: ExpandProblem) -> int:
    out = ctypes.c_size_t(0)
    rc = load_library().dispatch_expand_workspace_size(ctypes.byref(problem), ctypes.byref(out))
    if rc:
        raise DispatchError(rc, "dispatch_expand_workspace_size")
    return int(out.value)


@dataclasses.dataclass
class ExpandLayoutTensors:
    """Device int32 outputs of dispatch_expand_layout."""

    expert_count: torch.Tensor        # [E/R]
    expert_psum: torch.Tensor         # [E/R + 1]
    expert_slot: torch.Tensor         # [S*M, K]
    recv_src_row_idx: torch.Tensor    # [recv_capacity_rows]
    status: torch.Tensor              # [1]

    def ptrs(self, expert_count_cumulative: Optional[torch.Tensor] = None) -> LayoutPtrs:
        return LayoutPtrs(self.expert_count.data_ptr(), None, self.expert_psum.data_ptr(), None,
                          self.expert_slot.data_ptr(), None, self.recv_src_row_idx.data_ptr(), None,
                          self.status.data_ptr(), _ptr(expert_count_cumulative))


def alloc_expand_layout(problem: ExpandProblem, device) -> ExpandLayoutTensors:
    i32 = dict(dtype=torch.int32, device=device)
    local = problem.num_experts // problem.num_ranks
    rows = problem.num_sources * problem.rows_per_source
    return ExpandLayoutTensors(
        expert_count=torch.empty(local, **i32), expert_psum=torch.empty(local + 1, **i32),
        expert_slot=torch.empty((rows, problem.num_topk), **i32),
        recv_src_row_idx=torch.empty(max(problem.recv_capacity_rows, 1), **i32),
        status=torch.empty(1, **i32))


def alloc_expand_workspace(problem: ExpandProblem, device) -> torch.Tensor:
    """Workspace for the expand layout calls: zero-filled, as its first use requires."""
    n = dispatch_expand_workspace_size(problem)
    return torch.zeros((n + 255) // 256 * 256, dtype=torch.uint8, device=device)


def dispatch_expand_layout(problem: ExpandProblem, recv_topk_idx: torch.Tensor, recv_count: torch.Tensor,
                           out: ExpandLayoutTensors, workspace: torch.Tensor,
                           stream: Optional[torch.cuda.Stream] = None,
                           expert_count_cumulative: Optional[torch.Tensor] = None) -> None:
    """Enqueue the receiver's expert-major layout of a receive buffer. When
    ``expert_count_cumulative`` (device int32 [E/R], kept by the caller) is
    given, a successful call adds the local experts' received rows to it."""
    _check_device_tensor(recv_topk_idx, "recv_topk_idx")
    if recv_topk_idx.element_size() != problem.topk_idx_bytes:
        raise ValueError("recv_topk_idx element width does not match problem.topk_idx_bytes")
    _check_device_tensor(recv_count, "recv_count", torch.int32)
    _check_device_tensor(workspace, "workspace")
    for name, t in _fields_of(out):
        _check_device_tensor(t, name, torch.int32)
    _check_cumulative(expert_count_cumulative, problem.num_experts // problem.num_ranks)
    _check_expand_sizes(problem, recv_topk_idx, recv_count, out, None, None, None, None)
    lay = out.ptrs(expert_count_cumulative)
    rc = load_library().dispatch_expand_layout(
        ctypes.byref(problem), _ptr(recv_topk_idx), _ptr(recv_count), ctypes.byref(lay), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream, recv_topk_idx.device))
    if rc:
        raise DispatchError(rc, "dispatch_expand_layout")


def dispatch_expand_layout_and_scatter(problem: ExpandProblem, recv_topk_idx: torch.Tensor,
                                       recv_count: torch.Tensor, out: ExpandLayoutTensors, workspace: torch.Tensor,
                                       recv_buf: torch.Tensor, recv_sf_buf: Optional[torch.Tensor],
                                       recv_x: torch.Tensor, recv_sf: Optional[torch.Tensor],
                                       stream: Optional[torch.cuda.Stream] = None,
                                       expert_count_cumulative: Optional[torch.Tensor] = None) -> None:
    """Enqueue dispatch_expand_layout then dispatch_expand_scatter as one call
    (one kernel for a small receive buffer)."""
    _check_device_tensor(recv_topk_idx, "recv_topk_idx")
    if recv_topk_idx.element_size() != problem.topk_idx_bytes:
        raise ValueError("recv_topk_idx element width does not match problem.topk_idx_bytes")
    _check_device_tensor(recv_count, "recv_count", torch.int32)
    _check_device_tensor(workspace, "workspace")
    for name, t in _fields_of(out):
        _check_device_tensor(t, name, torch.int32)
    _check_cumulative(expert_count_cumulative, problem.num_experts // problem.num_ranks)
    _check_device_tensor(recv_buf, "recv_buf")
    for name, t in (("recv_sf_buf", recv_sf_buf), ("recv_x", recv_x), ("recv_sf", recv_sf)):
        if t is not None:
            _check_device_tensor(t, name)
    _check_expand_sizes(problem, recv_topk_idx, recv_count, out, recv_buf, recv_sf_buf, recv_x, recv_sf)
    lay = out.ptrs(expert_count_cumulative)
    rc = load_library().dispatch_expand_layout_and_scatter(
        ctypes.byref(problem), _ptr(recv_topk_idx), _ptr(recv_count), ctypes.byref(lay), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(recv_buf), _ptr(recv_sf_buf), _ptr(recv_x), _ptr(recv_sf),
        _stream_handle(stream, recv_topk_idx.device))
    if rc:
        raise DispatchError(rc, "dispatch_expand_layout_and_scatter")


def dispatch_expand_scatter(problem: ExpandProblem, layout: ExpandLayoutTensors, recv_buf: torch.Tensor,
                            recv_sf_buf: Optional[torch.Tensor], recv_x: torch.Tensor,
                            recv_sf: Optional[torch.Tensor], stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueue the copy of received rows into the expert-major buffer."""
    _check_device_tensor(recv_buf, "recv_buf")
    for name, t in (("recv_sf_buf", recv_sf_buf), ("recv_x", recv_x), ("recv_sf", recv_sf)):
        if t is not None:
            _check_device_tensor(t, name)
    for name, t in _fields_of(layout):
        _check_device_tensor(t, name, torch.int32)
    _check_expand_sizes(problem, None, None, layout, recv_buf, recv_sf_buf, recv_x, recv_sf)
    lay = layout.ptrs()
    rc = load_library().dispatch_expand_scatter(ctypes.byref(problem), ctypes.byref(lay), _ptr(recv_buf),
                                                _ptr(recv_sf_buf), _ptr(recv_x), _ptr(recv_sf),
                                                _stream_handle(stream, recv_buf.device))
    if rc:
        raise DispatchError(rc, "dispatch_expand_scatter")


class ExpandPlan:
    """A prepared receiver-side expand, like Plan: the tensors and the stream
    are checked once and the C arguments built once. ``layout()`` enqueues
    dispatch_expand_layout, ``scatter()`` dispatch_expand_scatter and
    ``__call__`` both as one dispatch_expand_layout_and_scatter call."""

    def __init__(self, problem: ExpandProblem, recv_topk_idx: torch.Tensor, recv_count: torch.Tensor,
                 layout: ExpandLayoutTensors, workspace: torch.Tensor, recv_buf: torch.Tensor,
                 recv_sf_buf: Optional[torch.Tensor], recv_x: torch.Tensor, recv_sf: Optional[torch.Tensor],
                 stream: Optional[torch.cuda.Stream] = None,
                 expert_count_cumulative: Optional[torch.Tensor] = None):
        _check_device_tensor(recv_topk_idx, "recv_topk_idx")
        if recv_topk_idx.element_size() != problem.topk_idx_bytes:
            raise ValueError("recv_topk_idx element width does not match problem.topk_idx_bytes")
        _check_device_tensor(recv_count, "recv_count", torch.int32)
        _check_device_tensor(workspace, "workspace")
        for name, t in _fields_of(layout):
            _check_device_tensor(t, name, torch.int32)
        _check_cumulative(expert_count_cumulative, problem.num_experts // problem.num_ranks)
        _check_device_tensor(recv_buf, "recv_buf")
        for name, t in (("recv_sf_buf", recv_sf_buf), ("recv_x", recv_x), ("recv_sf", recv_sf)):
            if t is not None:
                _check_device_tensor(t, name)
        _check_expand_sizes(problem, recv_topk_idx, recv_count, layout, recv_buf, recv_sf_buf, recv_x, recv_sf)
        # Its own copy of the problem, as in Plan.
        problem = ExpandProblem.from_buffer_copy(problem)
        self._problem = problem
        self._lib = load_library()
        self._keep = (problem, recv_topk_idx, recv_count, layout, workspace, recv_buf, recv_sf_buf, recv_x, recv_sf,
                      expert_count_cumulative)
        self._lay = layout.ptrs(expert_count_cumulative)
        handle = _stream_handle(stream, recv_topk_idx.device)
        rows = (_ptr(recv_buf), _ptr(recv_sf_buf), _ptr(recv_x), _ptr(recv_sf))
        self._layout_args = (ctypes.byref(problem), _ptr(recv_topk_idx), _ptr(recv_count), ctypes.byref(self._lay),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), handle)
        self._scatter_args = (ctypes.byref(problem), ctypes.byref(self._lay), *rows, handle)
        self._both_args = (*self._layout_args[:-1], *rows, handle)

    def layout(self) -> None:
        rc = self._lib.dispatch_expand_layout(*self._layout_args)
        if rc:
            raise DispatchError(rc, "dispatch_expand_layout")

    def scatter(self) -> None:
        rc = self._lib.dispatch_expand_scatter(*self._scatter_args)
        if rc:
            raise DispatchError(rc, "dispatch_expand_scatter")

    def __call__(self) -> None:
        rc = self._lib.dispatch_expand_layout_and_scatter(*self._both_args)
        if rc:
            raise DispatchError(rc, "dispatch_expand_layout_and_scatter")


# ------------------------------------------------------------------- combine


def dispatch_combine(expert_slot: torch.Tensor, topk_weights: torch.Tensor, y: torch.Tensor,
                     out: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueue out[t] = sum_k topk_weights[t, k] * y[expert_slot[t, k]] (bf16 rows, fp32 sums)."""
    _check_device_tensor(expert_slot, "expert_slot", torch.int32)
    _check_device_tensor(topk_weights, "topk_weights", torch.float32)
    _check_device_tensor(y, "y", torch.bfloat16)
    _check_device_tensor(out, "out", torch.bfloat16)
    t, k = expert_slot.shape
    if topk_weights.shape != (t, k) or out.shape[0] != t or out.shape[1] != y.shape[1]:
        raise ValueError("combine: shapes do not line up")
    problem = CombineProblem(t, k, 0, y.shape[1], y.shape[0])
    rc = load_library().dispatch_combine(ctypes.byref(problem), _ptr(expert_slot), _ptr(topk_weights), _ptr(y),
                                         _ptr(out), _stream_handle(stream, y.device))
    if rc:
        raise DispatchError(rc, "dispatch_combine")


class CombinePlan:
    """A prepared combine: the tensors and the stream are checked once and the
    C arguments built once, so each call is a single C call."""

    def __init__(self, expert_slot: torch.Tensor, topk_weights: torch.Tensor, y: torch.Tensor, out: torch.Tensor,
                 stream: Optional[torch.cuda.Stream] = None):
        _check_device_tensor(expert_slot, "expert_slot", torch.int32)
        _check_device_tensor(topk_weights, "topk_weights", torch.float32)
        _check_device_tensor(y, "y", torch.bfloat16)
        _check_device_tensor(out, "out", torch.bfloat16)
        t, k = expert_slot.shape
        if topk_weights.shape != (t, k) or out.shape[0] != t or out.shape[1] != y.shape[1]:
            raise ValueError("combine: shapes do not line up")
        self._lib = load_library()
        self._problem = CombineProblem(t, k, 0, y.shape[1], y.shape[0])
        self._keep = (expert_slot, topk_weights, y, out)
        self._args = (ctypes.byref(self._problem), _ptr(expert_slot), _ptr(topk_weights), _ptr(y), _ptr(out),
                      _stream_handle(stream, y.device))

    def __call__(self) -> None:
        rc = self._lib.dispatch_combine(*self._args)
        if rc:
            raise DispatchError(rc, "dispatch_combine")
