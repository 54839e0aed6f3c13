"""CPU oracle for MoE dispatch layout and scatter: TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``dispatch_oracle.c``: plain single-threaded C that
follows the "DeepEP Counting Sort / Bucketization" page step by step (Count,
Prefix Sum with alignment, rank- and expert-level slot scatter, row copies with
zero padding). Only ``tests/``, the smoke check and the benchmark's CPU
baseline may import this package; the product library never does, and the two
share no code.

Every function here is marshalling: numpy arrays in, the C oracle does the
arithmetic, numpy arrays out.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dispatch_oracle.c")
LIB_PATH = os.path.join(_HERE, "libdispatch_oracle.so")

BAD_EXPERT = 1
RECV_OVERFLOW = 2
RANK_OVERFLOW = 4
DUP_EXPERT = 8
BAD_COUNT = 16

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (single-threaded, -O2)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                    "-I", _HERE, "-o", tmp, src], check=True)
    os.replace(tmp, out)
    return out


def load_library(path: str):
    """Load a compiled oracle from ``path`` (the default build, or a test's variant)."""
    lib = ctypes.CDLL(path)
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_dispatch_layout.argtypes = [i64, i32, i32, i32, i32, p, i64, i64,
                                           p, p, p, p, p, p, p, p]
    lib.oracle_dispatch_layout.restype = ctypes.c_int
    lib.oracle_dispatch_scatter.argtypes = [i64, i32, i32, i64, i32, p, p, p, p, p, p,
                                            p, p, p, p, ctypes.c_int]
    lib.oracle_dispatch_scatter.restype = ctypes.c_int
    lib.oracle_expand_layout.argtypes = [i32, i32, i32, i32, i32, i32, i32, p, p, i64, p, p, p, p]
    lib.oracle_expand_layout.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [i64, i32, i64, i64, p, p, p, p]
    lib.oracle_combine.restype = ctypes.c_int
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load_library(LIB_PATH)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# Value the wrappers put in inverse-map entries beyond the totals, so a test
# can see that nothing past the totals was written.
CANARY = -7


@dataclasses.dataclass
class Layout:
    status: int
    num_experts: int
    num_ranks: int
    alignment: int
    expert_count: np.ndarray        # int32 [E]
    rank_count: np.ndarray          # int32 [R]
    expert_psum: np.ndarray         # int32 [E+1], exclusive, aligned
    rank_psum: np.ndarray           # int32 [R+1], exclusive
    expert_slot: np.ndarray         # int32 [T, K]
    rank_slot: np.ndarray           # int32 [T, K]
    recv_src_token_idx: np.ndarray  # int32 [recv_capacity]
    rank_src_token_idx: np.ndarray  # int32 [rank_capacity]

    @property
    def num_recv_rows(self) -> int:
        return int(self.expert_psum[-1])

    @property
    def num_rank_rows(self) -> int:
        return int(self.rank_psum[-1])


def max_rows(num_tokens: int, num_topk: int, num_experts: int, num_ranks: int,
             alignment: int) -> tuple:
    """Worst-case row counts: every pair routed, every expert padded by A-1."""
    return (num_tokens * num_topk + num_experts * (max(alignment, 1) - 1),
            num_tokens * min(num_topk, num_ranks))


def layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int, alignment: int = 1,
           recv_capacity: Optional[int] = None, rank_capacity: Optional[int] = None,
           lib=None) -> Layout:
    """Counts, psums, slot maps and inverse maps of one routing table."""
    lib = _load(lib)
    topk = np.ascontiguousarray(topk_idx, dtype=np.int64)
    if topk.ndim != 2:
        raise ValueError("topk_idx must be [T, K]")
    t, k = topk.shape
    mr, mk = max_rows(t, k, num_experts, num_ranks, alignment)
    recv_capacity = mr if recv_capacity is None else recv_capacity
    rank_capacity = mk if rank_capacity is None else rank_capacity
    out = Layout(
        status=0, num_experts=num_experts, num_ranks=num_ranks, alignment=alignment,
        expert_count=np.zeros(num_experts, np.int32), rank_count=np.zeros(num_ranks, np.int32),
        expert_psum=np.zeros(num_experts + 1, np.int32), rank_psum=np.zeros(num_ranks + 1, np.int32),
        expert_slot=np.full((t, k), CANARY, np.int32), rank_slot=np.full((t, k), CANARY, np.int32),
        recv_src_token_idx=np.full(max(recv_capacity, 0), CANARY, np.int32),
        rank_src_token_idx=np.full(max(rank_capacity, 0), CANARY, np.int32))
    rc = lib.oracle_dispatch_layout(
        t, k, num_experts, num_ranks, alignment, _ptr(topk), recv_capacity, rank_capacity,
        _ptr(out.expert_count), _ptr(out.rank_count), _ptr(out.expert_psum), _ptr(out.rank_psum),
        _ptr(out.expert_slot), _ptr(out.rank_slot), _ptr(out.recv_src_token_idx),
        _ptr(out.rank_src_token_idx))
    if rc < 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    out.status = rc
    return out


@dataclasses.dataclass
class ExpandLayout:
    status: int
    local_experts: int
    alignment: int
    expert_count: np.ndarray      # int32 [E/R]
    expert_psum: np.ndarray       # int32 [E/R + 1]
    expert_slot: np.ndarray       # int32 [S*M, K]
    recv_src_row_idx: np.ndarray  # int32 [recv_capacity]

    @property
    def num_recv_rows(self) -> int:
        return int(self.expert_psum[-1])


def expand_max_rows(num_sources: int, rows_per_source: int, num_topk: int, num_experts: int,
                    num_ranks: int, alignment: int) -> int:
    local = num_experts // num_ranks
    return num_sources * rows_per_source * min(num_topk, local) + local * (max(alignment, 1) - 1)


def expand_layout(recv_topk: np.ndarray, recv_count: np.ndarray, num_sources: int, rows_per_source: int,
                  num_experts: int, num_ranks: int, local_rank: int, alignment: int = 1,
                  recv_capacity: Optional[int] = None, lib=None) -> ExpandLayout:
    """Receiver-side expand layout over the local experts of `local_rank`."""
    lib = _load(lib)
    topk = np.ascontiguousarray(recv_topk, dtype=np.int64)
    counts = np.ascontiguousarray(recv_count, dtype=np.int32)
    rows, k = topk.shape
    if rows != num_sources * rows_per_source or counts.shape != (num_sources,):
        raise ValueError("recv_topk must be [S*M, K] and recv_count [S]")
    local = num_experts // num_ranks
    cap = expand_max_rows(num_sources, rows_per_source, k, num_experts, num_ranks, alignment) \
        if recv_capacity is None else recv_capacity
    out = ExpandLayout(
        status=0, local_experts=local, alignment=alignment,
        expert_count=np.zeros(local, np.int32), expert_psum=np.zeros(local + 1, np.int32),
        expert_slot=np.full((rows, k), CANARY, np.int32),
        recv_src_row_idx=np.full(max(cap, 0), CANARY, np.int32))
    rc = lib.oracle_expand_layout(num_sources, rows_per_source, k, num_experts, num_ranks, local_rank,
                                  alignment, _ptr(topk), _ptr(counts), cap, _ptr(out.expert_count),
                                  _ptr(out.expert_psum), _ptr(out.expert_slot), _ptr(out.recv_src_row_idx))
    if rc < 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    out.status = rc
    return out


@dataclasses.dataclass
class Rows:
    rank_x: Optional[np.ndarray]    # uint8 [N_r, row_bytes]
    rank_sf: Optional[np.ndarray]   # float32 [N_r, S]
    recv_x: Optional[np.ndarray]    # uint8 [P, row_bytes]
    recv_sf: Optional[np.ndarray]   # float32 [P, S]


def scatter(lay: Layout, x_bytes: np.ndarray, x_sf: Optional[np.ndarray] = None,
            rank_contig: bool = True, expert_major: bool = True, zero_pad: bool = True,
            fill: int = 0xA5, lib=None) -> Rows:
    """Rank-contiguous and expert-major row copies of one layout.

    Output rows are pre-filled with ``fill`` so that unwritten bytes are visible.
    """
    if lay.status != 0:
        raise ValueError("layout carries an error status; rows are unspecified")
    lib = _load(lib)
    x_bytes = np.ascontiguousarray(x_bytes, dtype=np.uint8)
    t, row_bytes = x_bytes.shape
    k = lay.expert_slot.shape[1]
    s = 0 if x_sf is None else int(x_sf.shape[1])
    sf = None if x_sf is None else np.ascontiguousarray(x_sf, dtype=np.float32)
    n_rank, n_recv = lay.num_rank_rows, lay.num_recv_rows

    def rows(n, width, dtype, on):
        if not on:
            return None
        a = np.empty((n, width), dtype=dtype)
        a.view(np.uint8)[...] = fill
        return a

    out = Rows(rank_x=rows(n_rank, row_bytes, np.uint8, rank_contig),
               rank_sf=rows(n_rank, s, np.float32, rank_contig and s > 0),
               recv_x=rows(n_recv, row_bytes, np.uint8, expert_major),
               recv_sf=rows(n_recv, s, np.float32, expert_major and s > 0))
    rc = lib.oracle_dispatch_scatter(
        t, k, lay.num_experts, row_bytes, s, _ptr(x_bytes), _ptr(sf),
        _ptr(lay.expert_count), _ptr(lay.expert_psum), _ptr(lay.expert_slot),
        _ptr(lay.rank_slot), _ptr(out.rank_x), _ptr(out.rank_sf), _ptr(out.recv_x),
        _ptr(out.recv_sf), 1 if zero_pad else 0)
    if rc != 0:
        raise ValueError(f"oracle scatter failed (code {rc})")
    return out


class Prepared:
    """The oracle's layout + scatter of one input, on pre-allocated, pre-faulted
    host buffers, for timing the oracle as it stands (the CPU baseline)."""

    def __init__(self, topk_idx: np.ndarray, num_experts: int, num_ranks: int, alignment: int,
                 x_bytes: np.ndarray, x_sf: Optional[np.ndarray] = None):
        self.lib = _load()
        self.topk = np.ascontiguousarray(topk_idx, dtype=np.int64)
        self.t, self.k = self.topk.shape
        self.e, self.r, self.a = num_experts, num_ranks, alignment
        self.x = np.ascontiguousarray(x_bytes, dtype=np.uint8)
        self.row_bytes = self.x.shape[1]
        self.sf = None if x_sf is None else np.ascontiguousarray(x_sf, dtype=np.float32)
        self.s = 0 if x_sf is None else self.sf.shape[1]
        self.recv_cap, self.rank_cap = max_rows(self.t, self.k, num_experts, num_ranks, alignment)
        z = lambda *shape, dt=np.int32: np.ones(shape, dtype=dt)  # noqa: E731  (ones: pre-faulted)
        self.expert_count, self.rank_count = z(num_experts), z(num_ranks)
        self.expert_psum, self.rank_psum = z(num_experts + 1), z(num_ranks + 1)
        self.expert_slot, self.rank_slot = z(self.t, self.k), z(self.t, self.k)
        self.recv_src, self.rank_src = z(self.recv_cap), z(self.rank_cap)
        self.rank_x = z(self.rank_cap, self.row_bytes, dt=np.uint8)
        self.recv_x = z(self.recv_cap, self.row_bytes, dt=np.uint8)
        self.rank_sf = z(self.rank_cap, self.s, dt=np.float32) if self.s else None
        self.recv_sf = z(self.recv_cap, self.s, dt=np.float32) if self.s else None

    def run_layout(self) -> int:
        return self.lib.oracle_dispatch_layout(
            self.t, self.k, self.e, self.r, self.a, _ptr(self.topk), self.recv_cap, self.rank_cap,
            _ptr(self.expert_count), _ptr(self.rank_count), _ptr(self.expert_psum), _ptr(self.rank_psum),
            _ptr(self.expert_slot), _ptr(self.rank_slot), _ptr(self.recv_src), _ptr(self.rank_src))

    def run_scatter(self) -> int:
        return self.lib.oracle_dispatch_scatter(
            self.t, self.k, self.e, self.row_bytes, self.s, _ptr(self.x), _ptr(self.sf),
            _ptr(self.expert_count), _ptr(self.expert_psum), _ptr(self.expert_slot), _ptr(self.rank_slot),
            _ptr(self.rank_x), _ptr(self.rank_sf), _ptr(self.recv_x), _ptr(self.recv_sf), 1)


def expand_scatter(lay: ExpandLayout, recv_buf: np.ndarray, recv_sf: Optional[np.ndarray] = None,
                   zero_pad: bool = True, fill: int = 0xA5, lib=None) -> Rows:
    """Expert-major rows of a receiver-side expand: the oracle's row copy over
    the receive buffer seen as S*M rows (no rank-contiguous output)."""
    if lay.status != 0:
        raise ValueError("layout carries an error status; rows are unspecified")
    lib = _load(lib)
    buf = np.ascontiguousarray(recv_buf, dtype=np.uint8)
    rows, row_bytes = buf.shape
    k = lay.expert_slot.shape[1]
    s = 0 if recv_sf is None else int(recv_sf.shape[1])
    sf = None if recv_sf is None else np.ascontiguousarray(recv_sf, dtype=np.float32)
    n = lay.num_recv_rows
    recv_x = np.empty((n, row_bytes), dtype=np.uint8)
    recv_x[...] = fill
    out_sf = None
    if s:
        out_sf = np.empty((n, s), dtype=np.float32)
        out_sf.view(np.uint8)[...] = fill
    no_rank = np.full(lay.expert_slot.shape, -1, dtype=np.int32)
    rc = lib.oracle_dispatch_scatter(
        rows, k, lay.local_experts, row_bytes, s, _ptr(buf), _ptr(sf), _ptr(lay.expert_count),
        _ptr(lay.expert_psum), _ptr(lay.expert_slot), _ptr(no_rank), None, None, _ptr(recv_x), _ptr(out_sf),
        1 if zero_pad else 0)
    if rc != 0:
        raise ValueError(f"oracle scatter failed (code {rc})")
    return Rows(rank_x=None, rank_sf=None, recv_x=recv_x, recv_sf=out_sf)


def combine(y_bits: np.ndarray, weights: np.ndarray, expert_slot: np.ndarray, lib=None) -> np.ndarray:
    """out[t] = sum_k weights[t, k] * y[expert_slot[t, k]] in double precision.

    y_bits: uint16 [rows, H] bf16 bit patterns; weights: float32 [T, K];
    expert_slot: int32 [T, K] (-1 = no contribution). Returns float64 [T, H].
    """
    lib = _load(lib)
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    slots = np.ascontiguousarray(expert_slot, dtype=np.int32)
    t, k = slots.shape
    rows, hidden = y.shape
    out = np.empty((t, hidden), dtype=np.float64)
    rc = lib.oracle_combine(t, k, hidden, rows, _ptr(y), _ptr(w), _ptr(slots), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle combine rejected the arguments (code {rc})")
    return out
