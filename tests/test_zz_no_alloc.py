"""The allocation-free entry point against the one it varies.

dispatch_layout_and_scatter_noalloc keeps the layout's workspace in the
library's own device array; every output must equal dispatch_layout_and_scatter's
with a caller workspace, bit for bit, on two calls in a row (the second smaller,
so it runs on what the first left in the array)."""

import dataclasses

import pytest
import torch

import moe_token_dispatch_amd as M
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _prepare(w):
    inp = W.make_inputs(w)
    t, k = inp.topk_idx.shape
    s = w.sf_per_token
    prob = M.make_problem(t, k, w.num_experts, w.num_ranks, w.alignment, 8, w.row_bytes, s)
    topk = torch.from_numpy(inp.topk_idx).to(H.DEVICE)
    x = inp.x.view(torch.uint8).to(H.DEVICE)
    sf = None if inp.x_sf is None else torch.from_numpy(inp.x_sf).to(H.DEVICE)
    return prob, topk, x, sf


def _outputs(prob):
    lay = M.alloc_layout(prob, H.DEVICE)
    for f in dataclasses.fields(lay):
        getattr(lay, f.name).fill_(H.CANARY)
    rows = M.alloc_rows(prob, H.DEVICE)
    for f in dataclasses.fields(rows):
        buf = getattr(rows, f.name)
        if buf is not None:
            buf.view(torch.uint8).fill_(H.ROW_FILL)
    return lay, rows


def _assert_same(a_lay, a_rows, b_lay, b_rows):
    for f in dataclasses.fields(a_lay):
        assert torch.equal(getattr(a_lay, f.name), getattr(b_lay, f.name)), f.name
    for f in dataclasses.fields(a_rows):
        x, y = getattr(a_rows, f.name), getattr(b_rows, f.name)
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f.name


# Two calls in a row on one GPU: the full 4096 x 7168 bf16 batch, then a
# smaller aligned fp8 batch with scale factors (its workspace is smaller than
# what the first call left in the array; nothing of it may leak through).
CASES = [
    [W.get("dsv3_bf16"),
     W.Workload("noalloc_small", 1500, 1024, "fp8", True, 64, 8, 6, mask_frac=0.03, alignment=16, seed=31)],
    [W.Workload("noalloc_mid", 3000, 512, "bf16", False, 128, 16, 8, mask_frac=0.05, alignment=4, seed=32),
     W.Workload("noalloc_tiny", 200, 256, "bf16", False, 16, 4, 4, seed=33)],
]


@pytest.mark.parametrize("pair", CASES, ids=["dsv3_then_small_fp8", "mid_then_tiny"])
def test_noalloc_matches_workspace_call(pair):
    for w in pair:
        print(f"\n[noalloc] {w.describe()}", flush=True)
        prob, topk, x, sf = _prepare(w)
        ref_lay, ref_rows = _outputs(prob)
        ws = M.alloc_workspace(prob, H.DEVICE)
        M.dispatch_layout_and_scatter(prob, topk, ref_lay, ws, x, sf, ref_rows.rank_x, ref_rows.rank_sf,
                                      ref_rows.recv_x, ref_rows.recv_sf)
        lay, rows = _outputs(prob)
        M.dispatch_layout_and_scatter_noalloc(prob, topk, lay, x, sf, rows.rank_x, rows.rank_sf, rows.recv_x,
                                              rows.recv_sf)
        torch.cuda.synchronize()
        assert int(lay.status.item()) == 0
        _assert_same(ref_lay, ref_rows, lay, rows)
