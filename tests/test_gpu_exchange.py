"""The one-launch layout on the GPU: tiles that exchange their key counts
through the workspace inside one kernel ("DeepEP Counting Sort /
Bucketization" page, section 4.5's cross-tile merge, done without a central
workgroup), which the calls that read the token rows ahead take.

- One zero-filled workspace serves a sequence of problems of every layout
  geometry (one launch with 1, 2, 4 or 8 chunks per wavefront, two launches,
  the column scan, an expand layout), through every entry point; each result
  equals the oracle's, and after every call the exchange region at the start
  of the workspace reads zero again, whichever path ran.
- The wait guard: with a bound of one poll, tiles give up; the call then
  reports DISPATCH_STATUS_TIMEOUT (or, if every tile was in time, the exact
  result), and leaves the workspace ready: the next call with the default
  bound is exact.

Runs on an MI355X only (marked ``gpu``).
"""

import numpy as np
import pytest
import torch

import moe_token_dispatch_amd as M
import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

EXCHANGE_BYTES = (8192 + 1) * 8  # the exchange region: 8192 words and the control word


def _banner(msg):
    print(f"\n[gpu-exchange] {msg}", flush=True)


def _uniform(seed, t, k, e, mask):
    rng = np.random.default_rng([seed, 7])
    if k == 1:
        topk = rng.integers(0, e, (t, 1), dtype=np.int64)
    elif t > 100_000:  # k distinct experts per token, without sorting every row
        topk = np.argpartition(rng.random((t, e), dtype=np.float32), k, axis=1)[:, :k].astype(np.int64)
    else:
        topk = np.argsort(rng.random((t, e)), axis=1)[:, :k].astype(np.int64)
    m = rng.random((t, k)) < mask
    topk[m] = -1
    return topk


def _exchange_region_is_zero(ws: torch.Tensor) -> bool:
    return int(torch.count_nonzero(ws[:EXCHANGE_BYTES]).item()) == 0


# (T, K, E, R, A, row_bytes, S, kernels of the combined call: 2 = the
# one-launch layout and the scatter)
SHAPES = [
    (4096, 8, 256, 8, 1, 64, 0, 2),      # one launch, 8-wavefront tiles, 64 tiles; words summed 4 at a time
    (31744, 8, 256, 8, 1, 16, 0, 3),     # 248 tiles: words past the region, two launches
    (31745, 8, 256, 8, 4, 16, 3, 2),     # one launch, 16-wavefront tiles of 2 chunks; each word split alone
    (3841, 8, 4096, 1024, 1, 16, 0, 4),  # column scan
    (63489, 8, 256, 8, 1, 16, 0, 3),     # 4096 pairs per tile: past 12-bit counts, two launches
    (2500, 6, 64, 8, 128, 48, 2, 2),     # top-6 (lanes 60..63 idle), pad inverse-map entries; 8 at a time
    (16384, 8, 256, 8, 1, 16, 0, 2),     # one launch, 128-token tiles; 2 at a time
    (5000, 1, 16, 4, 3, 32, 0, 2),       # top-1, 512-token tiles
    (10000, 2, 16, 4, 1, 32, 0, 2),      # top-2, 256-token tiles
    (260000, 1, 256, 8, 1, 16, 0, 2),    # top-1, 2048-token tiles of 2 chunks
    (180000, 3, 256, 8, 2, 16, 0, 2),    # top-3 (lane 63 idle), 16-wavefront tiles of 4 chunks
]


def test_one_workspace_across_geometries_and_entry_points():
    probs = [M.make_problem(t, k, e, r, a, 8, rb, s) for t, k, e, r, a, rb, s, _ in SHAPES]
    ws = torch.zeros(max(M.dispatch_workspace_size(p) for p in probs) + 256, dtype=torch.uint8, device=H.DEVICE)
    for i, ((t, k, e, r, a, rb, s, kernels), prob) in enumerate(zip(SHAPES, probs)):
        assert M.dispatch_kernel_count(prob)[1] == kernels, (t, k, e, r)
        topk = _uniform(100 + i, t, k, e, 0.05)
        xb = H.random_rows(100 + i, t, rb)
        sf = np.random.default_rng([i, 3]).random((t, s), dtype=np.float32) if s else None
        ref = oracle.layout(topk, e, r, a)
        for mode in ("layout", "read_ahead", "combined"):
            _banner(f"T={t} K={k} E={e} R={r} A={a} row_bytes={rb} S={s} {mode}")
            run = H.run_gpu(topk, e, r, a, xb, sf, workspace=ws, combined=mode == "combined",
                            read_ahead=mode == "read_ahead")
            torch.cuda.synchronize()
            H.assert_layout_equal(run, ref)
            H.assert_rows_full(run, ref, xb, sf)
            assert _exchange_region_is_zero(ws), (t, k, e, r, mode)


def test_expand_layout_leaves_the_exchange_region_alone():
    """The expand's workspace has the same region at its start, and its
    layout (count and assign kernels) never writes it; a dispatch that takes
    the one-launch layout then runs on the same buffer."""
    q = M.make_expand_problem(4, 600, 8, 256, 8, 0, 1, 8, 64, 0)
    t, k, e, r = 2000, 8, 256, 8
    prob = M.make_problem(t, k, e, r, 1, 8, 64, 0)
    n = max(M.dispatch_expand_workspace_size(q), M.dispatch_workspace_size(prob))
    ws = torch.zeros(n + 256, dtype=torch.uint8, device=H.DEVICE)
    recv_topk = torch.from_numpy(_uniform(9, 4 * 600, 8, 256, 0.0)).to(H.DEVICE)
    recv_count = torch.tensor([600, 500, 0, 317], dtype=torch.int32, device=H.DEVICE)
    lay = M.alloc_expand_layout(q, H.DEVICE)
    for f in ("expert_count", "expert_psum", "expert_slot", "recv_src_row_idx"):
        getattr(lay, f).fill_(H.CANARY)
    M.dispatch_expand_layout(q, recv_topk, recv_count, lay, ws)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == 0
    assert _exchange_region_is_zero(ws)
    ref = oracle.expand_layout(recv_topk.cpu().numpy(), recv_count.cpu().numpy(), 4, 600, 256, 8, 0, 1)
    assert np.array_equal(lay.expert_count.cpu().numpy(), ref.expert_count)
    assert np.array_equal(lay.expert_psum.cpu().numpy(), ref.expert_psum)
    assert np.array_equal(lay.expert_slot.cpu().numpy().reshape(-1), ref.expert_slot.reshape(-1))
    p_rows = int(ref.expert_psum[-1])
    assert np.array_equal(lay.recv_src_row_idx.cpu().numpy()[:p_rows], ref.recv_src_row_idx[:p_rows])
    # The same buffer then serves a dispatch that takes the one-launch layout.
    assert M.dispatch_kernel_count(prob)[1] == 2
    topk = _uniform(10, t, k, e, 0.05)
    xb = H.random_rows(10, t, 64)
    run = H.run_gpu(topk, e, r, 1, xb, workspace=ws, combined=True)
    torch.cuda.synchronize()
    ref = oracle.layout(topk, e, r, 1)
    H.assert_layout_equal(run, ref)
    H.assert_rows_full(run, ref, xb, None)
    assert _exchange_region_is_zero(ws)


def test_wait_guard_reports_timeout_and_recovers():
    t, k, e, r, rb = 4096, 8, 256, 8, 256
    prob = M.make_problem(t, k, e, r, 1, 8, rb, 0)
    ws = M.alloc_workspace(prob, H.DEVICE)
    timeouts = 0
    try:
        M.dispatch_set_wait_limit(1)
        for i in range(6):
            _banner(f"wait bound 1 poll, call {i}")
            topk = _uniform(200 + i, t, k, e, 0.05)
            xb = H.random_rows(200 + i, t, rb)
            run = H.run_gpu(topk, e, r, 1, xb, workspace=ws, combined=True)
            torch.cuda.synchronize()
            st = run.status()
            assert st in (0, M.STATUS_TIMEOUT), st
            if st == 0:
                ref = oracle.layout(topk, e, r, 1)
                H.assert_layout_equal(run, ref)
                H.assert_rows_full(run, ref, xb, None)
            else:
                timeouts += 1
            assert _exchange_region_is_zero(ws)
    finally:
        M.dispatch_set_wait_limit(0)
    print(f"[gpu-exchange] calls that timed out with a one-poll bound: {timeouts} of 6", flush=True)
    _banner("default bound again")
    topk = _uniform(300, t, k, e, 0.05)
    xb = H.random_rows(300, t, rb)
    run = H.run_gpu(topk, e, r, 1, xb, workspace=ws, combined=True)
    torch.cuda.synchronize()
    ref = oracle.layout(topk, e, r, 1)
    H.assert_layout_equal(run, ref)
    H.assert_rows_full(run, ref, xb, None)
    assert _exchange_region_is_zero(ws)


@pytest.mark.parametrize("t,k,e,r", [(4096, 8, 256, 8), (31745, 8, 256, 8)])
def test_repeated_experts_keep_exact_counts(t, k, e, r):
    """A tile whose tokens all name one expert K times: the status reports
    the repeat, and the counts and psums the tiles exchanged still equal the
    oracle's, one count per (token, k) pair (the widest count a tile can
    publish)."""
    topk = _uniform(400, t, k, e, 0.05)
    tpt = 64 if t == 4096 else 256  # tokens per tile of these geometries
    topk[3 * tpt:4 * tpt, :] = 5
    ref = oracle.layout(topk, e, r, 1)
    assert ref.status == oracle.DUP_EXPERT
    prob = M.make_problem(t, k, e, r, 1, 8, 64, 0)
    assert M.dispatch_kernel_count(prob)[1] == 2  # the one-launch layout
    _banner(f"T={t}: tile 3 routes every pair to expert 5")
    run = H.run_gpu(topk, e, r, 1, H.random_rows(400, t, 64), combined=True)
    torch.cuda.synchronize()
    H.assert_layout_equal(run, ref)
