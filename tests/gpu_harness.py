"""Run the HIP dispatch path through the C ABI and compare it with the CPU oracle.

Test infrastructure: it calls the product only through the binding of
``include/moe_dispatch.h`` and the oracle only through ``oracle``; the two
never see each other's code.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import moe_token_dispatch_amd as M
import oracle

DEVICE = "cuda:0"
CANARY = -7
ROW_FILL = 0xA5

LAYOUT_FIELDS = ("expert_count", "rank_count", "expert_psum", "rank_psum", "expert_slot", "rank_slot")


@dataclasses.dataclass
class DeviceRun:
    problem: M.Problem
    layout: M.LayoutTensors
    rows: M.RowBuffers
    x: torch.Tensor
    x_sf: Optional[torch.Tensor]
    workspace: torch.Tensor

    def status(self) -> int:
        return int(self.layout.status.item())

    def host_layout(self) -> dict:
        return {name: t.cpu().numpy() for name, t in self.layout.tensors()}


def random_rows(seed: int, t: int, row_bytes: int) -> np.ndarray:
    return np.random.default_rng([seed, 99]).integers(0, 256, size=(t, row_bytes), dtype=np.uint8)


def run_gpu(topk: np.ndarray, num_experts: int, num_ranks: int, alignment: int,
            x_bytes: np.ndarray, x_sf: Optional[np.ndarray] = None, *, topk_bytes: int = 8,
            flags: int = M.ALL_OUTPUTS, recv_capacity: Optional[int] = None,
            rank_capacity: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
            scatter: bool = True, combined: bool = False, read_ahead: bool = False) -> DeviceRun:
    """Layout and scatter of one batch on the GPU: two calls, or with
    ``combined`` the single dispatch_layout_and_scatter call. ``read_ahead``:
    the two calls as dispatch_layout_read_ahead, then dispatch_scatter with
    the DISPATCH_ROWS_READ_AHEAD hint (the scatter's bounded-occupancy
    launch)."""
    t, k = topk.shape
    row_bytes = x_bytes.shape[1]
    s = 0 if x_sf is None else x_sf.shape[1]
    prob = M.make_problem(t, k, num_experts, num_ranks, alignment, topk_bytes, row_bytes, s,
                          recv_capacity, rank_capacity, flags)
    lay = M.alloc_layout(prob, DEVICE)
    for _, t_ in lay.tensors():
        t_.fill_(CANARY)
    ws = workspace if workspace is not None else M.alloc_workspace(prob, DEVICE)
    rows = M.alloc_rows(prob, DEVICE)
    for f in dataclasses.fields(rows):
        buf = getattr(rows, f.name)
        if buf is not None:
            buf.view(torch.uint8).fill_(ROW_FILL)
    np_dtype = np.int64 if topk_bytes == 8 else np.int32
    topk_d = torch.from_numpy(np.ascontiguousarray(topk.astype(np_dtype))).to(DEVICE)
    x_d = torch.from_numpy(np.ascontiguousarray(x_bytes)).to(DEVICE)
    sf_d = None if x_sf is None else torch.from_numpy(np.ascontiguousarray(x_sf, dtype=np.float32)).to(DEVICE)
    if combined:
        M.dispatch_layout_and_scatter(prob, topk_d, lay, ws, x_d, sf_d, rows.rank_x, rows.rank_sf, rows.recv_x,
                                      rows.recv_sf)
    elif read_ahead:
        M.dispatch_layout_read_ahead(prob, topk_d, lay, ws, x_d, sf_d)
        if scatter:
            hinted = M.Problem.from_buffer_copy(prob)
            hinted.flags |= M.ROWS_READ_AHEAD
            M.dispatch_scatter(hinted, lay, x_d, sf_d, rows.rank_x, rows.rank_sf, rows.recv_x, rows.recv_sf)
    else:
        M.dispatch_layout(prob, topk_d, lay, ws)
        if scatter:
            M.dispatch_scatter(prob, lay, x_d, sf_d, rows.rank_x, rows.rank_sf, rows.recv_x, rows.recv_sf)
    torch.cuda.synchronize()
    return DeviceRun(prob, lay, rows, x_d, sf_d, ws)


def assert_layout_equal(run: DeviceRun, ref: oracle.Layout):
    """Bit-exact comparison of every layout output, plus untouched canary bands."""
    got = run.host_layout()
    assert int(got["status"][0]) == ref.status, f"status {int(got['status'][0])} != oracle {ref.status}"
    for name in ("expert_count", "rank_count", "expert_psum", "rank_psum"):
        assert np.array_equal(got[name], getattr(ref, name)), name
    if ref.status != 0:
        return
    for name in ("expert_slot", "rank_slot"):
        assert np.array_equal(got[name].reshape(ref.expert_slot.shape), getattr(ref, name)), name
    p_total, n_rank = ref.num_recv_rows, ref.num_rank_rows
    assert np.array_equal(got["recv_src_token_idx"][:p_total], ref.recv_src_token_idx[:p_total]), "recv_src"
    assert np.array_equal(got["rank_src_token_idx"][:n_rank], ref.rank_src_token_idx[:n_rank]), "rank_src"
    assert np.all(got["recv_src_token_idx"][p_total:] == CANARY), "recv_src written past the total"
    assert np.all(got["rank_src_token_idx"][n_rank:] == CANARY), "rank_src written past the total"


def assert_rows_full(run: DeviceRun, ref: oracle.Layout, x_bytes: np.ndarray, x_sf: Optional[np.ndarray]):
    """Every row byte against the oracle's scatter, and untouched rows past the totals."""
    p = run.problem
    want = oracle.scatter(ref, x_bytes, x_sf, rank_contig=bool(p.flags & M.RANK_CONTIG),
                          expert_major=bool(p.flags & M.EXPERT_MAJOR),
                          zero_pad=bool(p.flags & M.ZERO_PAD), fill=ROW_FILL)
    p_total, n_rank = ref.num_recv_rows, ref.num_rank_rows
    pairs = (("rank_x", n_rank), ("rank_sf", n_rank), ("recv_x", p_total), ("recv_sf", p_total))
    for name, n in pairs:
        buf = getattr(run.rows, name)
        w = getattr(want, name)
        if buf is None:
            assert w is None or w.size == 0 or name.endswith("sf"), name
            continue
        g = buf.view(torch.uint8).cpu().numpy()
        assert np.array_equal(g[:n], w.view(np.uint8)), f"{name} rows differ from the oracle"
        assert np.all(g[n:] == ROW_FILL), f"{name} written past the total"


def assert_rows_sampled(run: DeviceRun, ref: oracle.Layout, x_bytes: np.ndarray, x_sf: Optional[np.ndarray],
                        n_samples: int = 2048, seed: int = 0):
    """Sampled rows against the oracle's row definition, computed one row at a time."""
    rng = np.random.default_rng(seed)
    p_total, n_rank = ref.num_recv_rows, ref.num_rank_rows
    checks = []
    if run.rows.recv_x is not None and p_total:
        idx = np.unique(np.concatenate([rng.integers(0, p_total, n_samples), [0, p_total - 1]]))
        src = ref.recv_src_token_idx[idx]
        checks.append(("recv", idx, src))
    if run.rows.rank_x is not None and n_rank:
        idx = np.unique(np.concatenate([rng.integers(0, n_rank, n_samples), [0, n_rank - 1]]))
        checks.append(("rank", idx, ref.rank_src_token_idx[idx]))
    for kind, idx, src in checks:
        xb = getattr(run.rows, f"{kind}_x")
        got = xb[torch.from_numpy(idx).to(DEVICE)].cpu().numpy()
        want = np.where((src >= 0)[:, None], x_bytes[np.maximum(src, 0)], 0).astype(np.uint8)
        assert np.array_equal(got, want), f"sampled {kind}_x rows differ from the oracle"
        sfb = getattr(run.rows, f"{kind}_sf")
        if x_sf is not None and sfb is not None:
            got = sfb[torch.from_numpy(idx).to(DEVICE)].view(torch.int32).cpu().numpy()
            xs = x_sf.view(np.int32)
            want = np.where((src >= 0)[:, None], xs[np.maximum(src, 0)], 0)
            assert np.array_equal(got, want), f"sampled {kind}_sf rows differ from the oracle"


def assert_rows_gather_property(run: DeviceRun, ref: oracle.Layout, chunk: int = 8192):
    """All rows, on the device: row s equals x[token of s] (a torch gather), pads are zero."""
    p_total, n_rank = ref.num_recv_rows, ref.num_rank_rows
    recv_src = torch.from_numpy(ref.recv_src_token_idx[:p_total].astype(np.int64)).to(DEVICE)
    rank_src = torch.from_numpy(ref.rank_src_token_idx[:n_rank].astype(np.int64)).to(DEVICE)
    x = run.x
    for lo in range(0, p_total, chunk):
        hi = min(p_total, lo + chunk)
        src = recv_src[lo:hi]
        real = src >= 0
        got = run.rows.recv_x[lo:hi]
        assert torch.equal(got[real], x.index_select(0, src[real])), f"recv_x rows {lo}..{hi}"
        assert not bool(got[~real].any()), f"recv_x pad rows {lo}..{hi} not zero"
        if run.x_sf is not None and run.rows.recv_sf is not None:
            gs = run.rows.recv_sf[lo:hi].view(torch.int32)
            assert torch.equal(gs[real], run.x_sf.view(torch.int32).index_select(0, src[real]))
            assert not bool(gs[~real].any())
    for lo in range(0, n_rank, chunk):
        hi = min(n_rank, lo + chunk)
        src = rank_src[lo:hi]
        assert torch.equal(run.rows.rank_x[lo:hi], x.index_select(0, src)), f"rank_x rows {lo}..{hi}"
        if run.x_sf is not None and run.rows.rank_sf is not None:
            assert torch.equal(run.rows.rank_sf[lo:hi].view(torch.int32),
                               run.x_sf.view(torch.int32).index_select(0, src))


# ------------------------------------------------------------------ combine
# The combine kernel widens bf16 to fp32, adds one fused multiply-add per
# routed k (ascending k, from 0) and rounds the fp32 sum to bf16 once. With
# A = sum_k |w_k| |y_k| and u = 2^-24, the K-term fp32 chain is within K u A of
# the exact sum S (each FMA rounds once, to at most u times a partial sum that
# is at most A), and the final rounding adds at most half a bf16 ulp,
# 2^-8 |S_fp32|. The accepted bound is
#     |gpu - S| <= 2^-8 (max(|gpu|, |S|) + (K+1) u A) + (K+1) u A + 2^-133
# (the last term covers bf16's subnormal spacing).

U = 2.0 ** -24


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bits, to nearest, ties to even, straight from the
    fp64 significand (no intermediate fp32 rounding). Normal range only."""
    m, e = np.frexp(v)                        # v = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)   # 8 significant bits, numpy rounds half to even
    return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def assert_combine_close(got_bits, y_bits, wts, slots, min_exact=0.99):
    """Combine output bits against the oracle's exact sums: every output
    within the bound above, at least `min_exact` of them equal to the exact
    sum rounded to bf16, and +0 rows for tokens with no routed entry."""
    s = oracle.combine(y_bits, wts, slots)
    a = oracle.combine(y_bits & np.uint16(0x7FFF), np.abs(wts), slots)
    k = slots.shape[1]
    got = bf16_bits_to_f64(got_bits)
    assert np.all(np.isfinite(got))
    err = (k + 1) * U * a
    bound = 2.0 ** -8 * (np.maximum(np.abs(got), np.abs(s)) + err) + err + 2.0 ** -133
    bad = np.abs(got - s) > bound
    assert not bad.any(), f"{int(bad.sum())} outputs outside the fp32-chain bound, first at {np.argwhere(bad)[0]}"
    exact = got_bits == f64_to_bf16_rne(s)
    assert exact.mean() >= min_exact, f"only {exact.mean():.5f} of outputs equal bf16(exact sum)"
    none = (slots < 0).all(axis=1)
    assert np.all(got_bits[none] == 0), "tokens with no routed entry must get +0 rows"
    return exact.mean()
