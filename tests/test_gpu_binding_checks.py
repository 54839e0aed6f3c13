"""The Python binding refuses tensors too small for the problem.

The C ABI takes raw pointers and trusts their sizes. The binding knows every
size from the problem, so a routing table, layout array, source row buffer
or output buffer one element short raises ValueError before anything is
enqueued. A correctly sized call then still succeeds.
"""

import dataclasses

import numpy as np
import pytest
import torch

import moe_token_dispatch_amd as M
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _short(t: torch.Tensor) -> torch.Tensor:
    """The same storage one element short (still contiguous)."""
    return t.reshape(-1)[:-1]


def test_dispatch_calls_refuse_undersized_tensors():
    t, k, e, r, a, rb, s = 100, 8, 64, 8, 4, 64, 2
    w = W.Workload("sizes", t, 32, "bf16", False, e, r, k, mask_frac=0.05, seed=5)
    topk = W.make_topk(w)
    prob = M.make_problem(t, k, e, r, a, 8, rb, s)
    lay, ws, rows = M.alloc_layout(prob, H.DEVICE), M.alloc_workspace(prob, H.DEVICE), M.alloc_rows(prob, H.DEVICE)
    topk_d = torch.from_numpy(topk).to(H.DEVICE)
    x = torch.zeros((t, rb), dtype=torch.uint8, device=H.DEVICE)
    sf = torch.zeros((t, s), dtype=torch.float32, device=H.DEVICE)
    rx, rsf, ex, esf = rows.rank_x, rows.rank_sf, rows.recv_x, rows.recv_sf

    with pytest.raises(ValueError, match="topk_idx"):
        M.dispatch_layout(prob, _short(topk_d), lay, ws)
    for f in dataclasses.fields(lay):
        small = dataclasses.replace(lay, **{f.name: _short(getattr(lay, f.name))}) if getattr(lay, f.name).numel() > 1 \
            else dataclasses.replace(lay, **{f.name: getattr(lay, f.name)[:0]})
        with pytest.raises(ValueError, match=f.name):
            M.dispatch_layout(prob, topk_d, small, ws)
        with pytest.raises(ValueError, match=f.name):
            M.dispatch_scatter(prob, small, x, sf, rx, rsf, ex, esf)
    for i, name in enumerate(("x", "x_sf", "rank_x", "rank_sf", "recv_x", "recv_sf")):
        args = [x, sf, rx, rsf, ex, esf]
        args[i] = _short(args[i])
        with pytest.raises(ValueError, match=name):
            M.dispatch_scatter(prob, lay, *args)
        with pytest.raises(ValueError, match=name):
            M.dispatch_layout_and_scatter(prob, topk_d, lay, ws, *args)
        with pytest.raises(ValueError, match=name):
            M.Plan(prob, topk_d, lay, ws, args[0], args[1], M.RowBuffers(*args[2:]))
    torch.cuda.synchronize()
    # Nothing ran: the layout still holds what it was allocated with, and a
    # correctly sized call works.
    M.dispatch_layout_and_scatter(prob, topk_d, lay, ws, x, sf, rx, rsf, ex, esf)
    torch.cuda.synchronize()
    ref = oracle.layout(topk, e, r, a)
    assert int(lay.status.item()) == 0
    assert np.array_equal(lay.expert_psum.cpu().numpy(), ref.expert_psum)


def test_expand_calls_refuse_undersized_tensors():
    s_count, m, k, e, r, rank, a, rb, sfw = 3, 20, 8, 64, 8, 2, 4, 64, 2
    q = M.make_expand_problem(s_count, m, k, e, r, rank, a, 8, rb, sfw)
    lay, ws = M.alloc_expand_layout(q, H.DEVICE), M.alloc_expand_workspace(q, H.DEVICE)
    cap = max(q.recv_capacity_rows, 1)
    topk = torch.full((s_count * m, k), -1, dtype=torch.int64, device=H.DEVICE)
    counts = torch.zeros(s_count, dtype=torch.int32, device=H.DEVICE)
    buf = torch.zeros((s_count * m, rb), dtype=torch.uint8, device=H.DEVICE)
    buf_sf = torch.zeros((s_count * m, sfw), dtype=torch.float32, device=H.DEVICE)
    rx = torch.zeros((cap, rb), dtype=torch.uint8, device=H.DEVICE)
    rsf = torch.zeros((cap, sfw), dtype=torch.float32, device=H.DEVICE)

    with pytest.raises(ValueError, match="recv_topk_idx"):
        M.dispatch_expand_layout(q, _short(topk), counts, lay, ws)
    with pytest.raises(ValueError, match="recv_count"):
        M.dispatch_expand_layout(q, topk, _short(counts), lay, ws)
    for f in dataclasses.fields(lay):
        small = dataclasses.replace(lay, **{f.name: _short(getattr(lay, f.name))}) if getattr(lay, f.name).numel() > 1 \
            else dataclasses.replace(lay, **{f.name: getattr(lay, f.name)[:0]})
        with pytest.raises(ValueError, match=f.name):
            M.dispatch_expand_layout(q, topk, counts, small, ws)
        with pytest.raises(ValueError, match=f.name):
            M.dispatch_expand_scatter(q, small, buf, buf_sf, rx, rsf)
    for i, name in enumerate(("recv_buf", "recv_sf_buf", "recv_x", "recv_sf")):
        args = [buf, buf_sf, rx, rsf]
        args[i] = _short(args[i])
        with pytest.raises(ValueError, match=name):
            M.dispatch_expand_scatter(q, lay, *args)
        with pytest.raises(ValueError, match=name):
            M.dispatch_expand_layout_and_scatter(q, topk, counts, lay, ws, *args)
        with pytest.raises(ValueError, match=name):
            M.ExpandPlan(q, topk, counts, lay, ws, *args)
    M.dispatch_expand_layout_and_scatter(q, topk, counts, lay, ws, buf, buf_sf, rx, rsf)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == 0
