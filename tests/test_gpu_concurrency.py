"""Calls running at the same time on several streams, through the C ABI.

The library keeps no state between calls, so calls that overlap on different
streams, each with its own workspace and outputs, must each give the oracle's
result for its own batch, bit for bit. One running per-expert count array is
shared by all of them: every successful call adds its counts with device
atomics, so the array ends at the sum over all calls.
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

# (tokens, alignment, one call, row bytes, scale factors per row): a batch of
# several layout tiles through the layout and scatter calls, a one-kernel
# batch through the one call, and a small batch at alignment 128 whose pad
# rows the scatter maps to row blocks.
CASES = [(3000, 1, False, 2048, 0), (200, 16, True, 1024, 4), (16, 128, False, 512, 4)]


def test_overlapping_calls_on_streams_share_only_the_running_counts():
    e, r, k, rounds = 256, 8, 8, 5
    cumulative = torch.zeros(e, dtype=torch.int32, device=H.DEVICE)
    jobs = []
    for i, (t, a, one_call, row_bytes, s) in enumerate(CASES):
        w = W.Workload(f"streams{i}", t, 64, "bf16", False, e, r, k, mask_frac=0.05, seed=700 + i)
        topk = W.make_topk(w)
        xb = H.random_rows(40 + i, t, row_bytes)
        sf = None if s == 0 else np.random.default_rng([i, 3]).uniform(0.5, 2, (t, s)).astype(np.float32)
        prob = M.make_problem(t, k, e, r, a, 8, row_bytes, s)
        lay, ws, rows = M.alloc_layout(prob, H.DEVICE), M.alloc_workspace(prob, H.DEVICE), M.alloc_rows(prob, H.DEVICE)
        for f in dataclasses.fields(lay):
            getattr(lay, f.name).fill_(H.CANARY)
        for f in dataclasses.fields(rows):
            buf = getattr(rows, f.name)
            if buf is not None:
                buf.view(torch.uint8).fill_(H.ROW_FILL)
        jobs.append(dict(topk=topk, xb=xb, sf=sf, prob=prob, lay=lay, ws=ws, rows=rows, one_call=one_call, a=a,
                         topk_d=torch.from_numpy(topk).to(H.DEVICE), x_d=torch.from_numpy(xb).to(H.DEVICE),
                         sf_d=None if sf is None else torch.from_numpy(sf).to(H.DEVICE),
                         stream=torch.cuda.Stream(device=H.DEVICE)))
    torch.cuda.synchronize()  # inputs and canaries are in place before any stream starts
    print(f"\n[gpu-streams] {len(jobs)} streams x {rounds} rounds", flush=True)
    for _ in range(rounds):
        for j in jobs:
            rows, st = j["rows"], j["stream"]
            if j["one_call"]:
                M.dispatch_layout_and_scatter(j["prob"], j["topk_d"], j["lay"], j["ws"], j["x_d"], j["sf_d"],
                                              rows.rank_x, rows.rank_sf, rows.recv_x, rows.recv_sf, stream=st,
                                              expert_count_cumulative=cumulative)
            else:
                M.dispatch_layout(j["prob"], j["topk_d"], j["lay"], j["ws"], stream=st,
                                  expert_count_cumulative=cumulative)
                M.dispatch_scatter(j["prob"], j["lay"], j["x_d"], j["sf_d"], rows.rank_x, rows.rank_sf, rows.recv_x,
                                   rows.recv_sf, stream=st)
    torch.cuda.synchronize()
    want = np.zeros(e, dtype=np.int64)
    for j in jobs:
        ref = oracle.layout(j["topk"], e, r, j["a"])
        assert ref.status == 0
        run = H.DeviceRun(j["prob"], j["lay"], j["rows"], j["x_d"], j["sf_d"], j["ws"])
        H.assert_layout_equal(run, ref)
        H.assert_rows_full(run, ref, j["xb"], j["sf"])
        want += rounds * ref.expert_count.astype(np.int64)
    assert np.array_equal(cumulative.cpu().numpy().astype(np.int64), want)
