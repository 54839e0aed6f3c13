"""GPU parity of dispatch_layout_and_scatter against the CPU oracle, bit for
bit, through the C ABI.

A small batch (up to 3072 (token, k) pairs, 2048 with pad rows, fewer with
many keys) is laid out
and copied by one kernel in which every workgroup ranks the whole batch itself
and copies its share of the rows' 1 KB segments; larger batches run the layout
and scatter kernels. Either way the outputs must equal
the oracle's layout and scatter: every count, psum, slot, inverse-map entry,
status bit and row byte, with canary bands past every total left untouched.
"""

import numpy as np
import pytest
import torch

import moe_token_dispatch_amd as M
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"\n[gpu-fused] {msg}", flush=True)


def _topk(seed, t, k, e, mask=0.0):
    w = W.Workload("fused", t, 64, "bf16", False, e, 1, k, mask_frac=mask, seed=seed)
    return W.make_topk(w)


def _fused(topk, e, r, a, row_bytes=64, s=0, seed=0, **kw):
    t = topk.shape[0]
    xb = H.random_rows(seed, t, row_bytes)
    sf = None if s == 0 else np.random.default_rng([seed, 7]).uniform(0.5, 2, (t, s)).astype(np.float32)
    ref = oracle.layout(topk, e, r, a, recv_capacity=kw.get("recv_capacity"), rank_capacity=kw.get("rank_capacity"))
    run = H.run_gpu(topk, e, r, a, xb, sf, combined=True, **kw)
    H.assert_layout_equal(run, ref)
    if ref.status == 0:
        H.assert_rows_full(run, ref, xb, sf)
    else:
        assert np.all(run.layout.expert_slot.cpu().numpy() == H.CANARY)
        for name in ("rank_x", "recv_x"):
            buf = getattr(run.rows, name)
            if buf is not None:
                assert np.all(buf.cpu().numpy() == H.ROW_FILL), name
    return run, ref


# One kernel up to 256 tokens at top-8 (one tile of 16 wavefronts x 2 chunks).
@pytest.mark.parametrize("t", [0, 1, 2, 7, 63, 64, 65, 128, 129, 200, 255, 256])
def test_token_counts_of_one_tile(t):
    _banner(f"T={t}")
    _fused(_topk(31, t, 8, 256, 0.05), 256, 8, 4, seed=t)


# The largest one-tile batch for each top-k: 16 x 2 x floor(64 / K) tokens,
# up to 8 tokens (and at most 32 pairs) per workgroup.
@pytest.mark.parametrize("k,t,e,r", [(1, 2048, 64, 8), (2, 1024, 64, 8), (3, 672, 64, 16), (5, 384, 64, 4),
                                     (7, 288, 128, 8), (16, 128, 64, 8), (32, 64, 64, 4)])
def test_largest_one_tile_batch_per_topk(k, t, e, r):
    _banner(f"K={k} T={t} E={e} R={r}")
    _fused(_topk(32 + k, t, k, e, 0.1), e, r, 3, row_bytes=48, seed=k)


# Rows of whole 1 KB units, rows whose last unit is partial (1040 and 2064 B),
# and rows shorter than one unit.
@pytest.mark.parametrize("row_bytes,s", [(16, 0), (4096, 0), (14336, 0), (7168, 56), (112, 1), (1040, 0),
                                         (2064, 3)])
def test_row_and_scale_factor_widths(row_bytes, s):
    _banner(f"row_bytes={row_bytes} S={s}")
    _fused(_topk(33, 256, 8, 256, 0.05), 256, 8, 1, row_bytes=row_bytes, s=s, seed=3)


def test_wide_pad_rows_with_scale_factors():
    """Alignment 128 on 7 KB rows with 56 scale factors: many zeroed pad rows."""
    _banner("A=128, 7168 B rows, S=56")
    _fused(_topk(43, 256, 8, 256, 0.05), 256, 8, 128, row_bytes=7168, s=56, seed=10)


@pytest.mark.parametrize("a", [1, 2, 3, 128])
def test_alignments(a):
    _banner(f"A={a}")
    _fused(_topk(34, 200, 8, 64, 0.05), 64, 8, a, row_bytes=80, s=3, seed=4)


@pytest.mark.parametrize("flags", [1, 2, 3, 6, 7])
def test_output_selection(flags):
    _banner(f"flags={flags}")
    _fused(_topk(35, 180, 8, 64, 0.05), 64, 8, 16, row_bytes=96, s=2, seed=5, flags=flags)


def test_int32_routing_and_fully_masked_tokens():
    _banner("int32 routing, masked tokens")
    topk = _topk(36, 230, 8, 256, 0.0)
    topk[::5] = -1
    topk[1::7, :5] = -3
    _fused(topk, 256, 8, 4, seed=6, topk_bytes=4)


# Past one layout tile, the one kernel ranks a tile of 4 (or, with few
# wavefronts, 8) chunks per wavefront, up to 3072 pairs without pad rows
# (with them, up to 2048).
@pytest.mark.parametrize("k,t,e,r", [(8, 257, 256, 8), (8, 300, 64, 8), (8, 384, 256, 8), (1, 3072, 64, 8),
                                     (2, 1536, 64, 4), (3, 1024, 64, 16)])
def test_batches_past_one_layout_tile(k, t, e, r):
    _banner(f"K={k} T={t} E={e} R={r}")
    prob = M.make_problem(t, k, e, r, 1, 8, 144, 2)
    assert M.dispatch_kernel_count(prob)[1] == 1
    _fused(_topk(42 + k, t, k, e, 0.05), e, r, 1, row_bytes=144, s=2, seed=t)


# With zero pad rows to write, the one kernel stops at 2048 pairs: 256 tokens
# at top-8 take it, 257 take the layout kernel (one launch: 5 tiles that
# exchange their counts) and the scatter kernel.
@pytest.mark.parametrize("t,kernels", [(256, 1), (257, 2)])
def test_pad_rows_limit_of_the_one_kernel(t, kernels):
    _banner(f"A=16 T={t}")
    prob = M.make_problem(t, 8, 256, 8, 16, 8, 144, 2)
    assert M.dispatch_kernel_count(prob)[1] == kernels
    _fused(_topk(44, t, 8, 256, 0.05), 256, 8, 16, row_bytes=144, s=2, seed=t)


def test_many_keys_eight_chunks_and_just_past_them():
    """E + R = 5120 keys leave room for 5 wavefronts of counters: the one
    kernel's tile holds 5 x 8 chunks x 8 tokens = 320 tokens at top-8; 321
    take the layout and scatter kernels."""
    for t in (80, 320, 321):
        _banner(f"E=4096 R=1024 T={t}")
        assert M.dispatch_kernel_count(M.make_problem(t, 8, 4096, 1024, 1, 8, 64, 0))[1] == (1 if t <= 320 else 3)
        _fused(_topk(37, t, 8, 4096, 0.05), 4096, 1024, 1, seed=t)


@pytest.mark.parametrize("t", [385, 3001])
def test_larger_batches_take_the_layout_and_scatter_kernels(t):
    _banner(f"T={t}")
    _fused(_topk(38, t, 8, 256, 0.05), 256, 8, 4, seed=t)


def test_status_bad_expert_writes_nothing():
    topk = _topk(39, 150, 4, 16)
    topk[77, 2] = 16
    _, ref = _fused(topk, 16, 4, 1, seed=7)
    assert ref.status == oracle.BAD_EXPERT


def test_status_capacity_overflow_writes_nothing():
    topk = _topk(40, 200, 8, 64)
    mr, mk = oracle.max_rows(200, 8, 64, 8, 4)
    full = oracle.layout(topk, 64, 8, 4)
    _, ref = _fused(topk, 64, 8, 4, seed=8, recv_capacity=full.num_recv_rows - 1, rank_capacity=mk)
    assert ref.status == oracle.RECV_OVERFLOW
    _, ref = _fused(topk, 64, 8, 4, seed=8, recv_capacity=mr, rank_capacity=full.num_rank_rows - 1)
    assert ref.status == oracle.RANK_OVERFLOW


def test_plan_call_and_running_counts():
    """A prepared plan's single call, twice, with the running per-expert counts."""
    _banner("plan call")
    t, k, e, r, a = 128, 8, 64, 8, 2
    topk = _topk(41, t, k, e, 0.05)
    xb = H.random_rows(9, t, 256)
    prob = M.make_problem(t, k, e, r, a, 8, 256, 0)
    lay, ws, rows = M.alloc_layout(prob, H.DEVICE), M.alloc_workspace(prob, H.DEVICE), M.alloc_rows(prob, H.DEVICE)
    for _, t_ in lay.tensors():  # canary bands past the totals, as assert_layout_equal expects
        t_.fill_(H.CANARY)
    cum = torch.zeros(e, dtype=torch.int32, device=H.DEVICE)
    plan = M.Plan(prob, torch.from_numpy(topk).to(H.DEVICE), lay, ws, torch.from_numpy(xb).to(H.DEVICE), None,
                  rows, expert_count_cumulative=cum)
    plan()
    plan()
    torch.cuda.synchronize()
    ref = oracle.layout(topk, e, r, a)
    run = H.DeviceRun(prob, lay, rows, torch.from_numpy(xb).to(H.DEVICE), None, ws)
    H.assert_layout_equal(run, ref)
    want = oracle.scatter(ref, xb)
    assert np.array_equal(rows.recv_x[:ref.num_recv_rows].cpu().numpy(), want.recv_x[:ref.num_recv_rows])
    assert np.array_equal(rows.rank_x[:ref.num_rank_rows].cpu().numpy(), want.rank_x[:ref.num_rank_rows])
    assert np.array_equal(cum.cpu().numpy(), 2 * ref.expert_count.astype(np.int64))
