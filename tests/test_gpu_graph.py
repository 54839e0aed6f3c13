"""A whole dispatch step (layout + scatter, and the combine for bf16 rows)
captured into a HIP graph and
replayed: every replay, on new routing and new rows copied into the captured
inputs, must match the CPU oracle bit for bit. The library launches kernels
only (no allocation, no memset, no synchronisation), so it can be captured.

Between replays the program does its own eager work (canary fills, input
copies) and synchronises, and each replay is checked on its own.
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


# The layout and scatter calls on a batch of several tiles, and the combined
# call on small batches, where it is one kernel.
@pytest.mark.parametrize("dtype,with_sf,alignment,t,combined", [
    ("bf16", False, 1, 1500, False), ("fp8", True, 16, 1500, False),
    ("bf16", False, 1, 200, True), ("fp8", True, 16, 300, True)])
def test_captured_dispatch_replays_match_oracle(dtype, with_sf, alignment, t, combined):
    print(f"\n[gpu-graph] capture dtype={dtype} sf={with_sf} A={alignment} T={t} combined={combined}", flush=True)
    base = W.Workload("graph", t, 512, dtype, with_sf, 64, 8, 8, mask_frac=0.05, alignment=alignment, seed=31)
    t, k, e, r = base.num_tokens, base.num_topk, base.num_experts, base.num_ranks
    prob = M.make_problem(t, k, e, r, alignment, 8, base.row_bytes, base.sf_per_token)
    lay = M.alloc_layout(prob, H.DEVICE)
    ws = M.alloc_workspace(prob, H.DEVICE)
    rows = M.alloc_rows(prob, H.DEVICE)
    topk_d = torch.zeros((t, k), dtype=torch.int64, device=H.DEVICE)
    x_d = torch.zeros((t, base.row_bytes), dtype=torch.uint8, device=H.DEVICE)
    sf_d = torch.zeros((t, base.sf_per_token), dtype=torch.float32, device=H.DEVICE) if with_sf else None

    def load(seed):
        w = dataclasses.replace(base, seed=seed)
        inp = W.make_inputs(w)
        topk_d.copy_(torch.from_numpy(inp.topk_idx))
        x_d.copy_(torch.from_numpy(inp.x_bytes()))
        if with_sf:
            sf_d.copy_(torch.from_numpy(inp.x_sf))
        for f in dataclasses.fields(lay):
            getattr(lay, f.name).fill_(H.CANARY)
        for f in dataclasses.fields(rows):
            buf = getattr(rows, f.name)
            if buf is not None:
                buf.view(torch.uint8).fill_(H.ROW_FILL)
        return inp

    # bf16 rows: the combine of the scattered rows joins the captured step.
    combine = dtype == "bf16"
    wts_d = torch.zeros((t, k), dtype=torch.float32, device=H.DEVICE)
    out_d = torch.zeros((t, base.hidden), dtype=torch.bfloat16, device=H.DEVICE)

    if combined:
        assert M.dispatch_kernel_count(prob)[1] == 1

    def step():
        if combined:
            M.dispatch_layout_and_scatter(prob, topk_d, lay, ws, x_d, sf_d, rows.rank_x, rows.rank_sf, rows.recv_x,
                                          rows.recv_sf)
        else:
            M.dispatch_layout(prob, topk_d, lay, ws)
            M.dispatch_scatter(prob, lay, x_d, sf_d, rows.rank_x, rows.rank_sf, rows.recv_x, rows.recv_sf)
        if combine:
            M.dispatch_combine(lay.expert_slot.view(t, k), wts_d, rows.recv_x.view(torch.bfloat16), out_d)

    side = torch.cuda.Stream(device=H.DEVICE)
    load(100)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream, outside the graph
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()

    for seed in (101, 102, 103, 102):
        inp = load(seed)
        wts = W.make_topk_weights(dataclasses.replace(base, seed=seed), inp.topk_idx)
        wts_d.copy_(torch.from_numpy(wts))
        out_d.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.layout(inp.topk_idx, e, r, alignment)
        run = H.GpuRun(prob, lay, rows, x_d, sf_d, ws)
        H.assert_layout_equal(run, ref)
        H.assert_rows_full(run, ref, inp.x_bytes(), inp.x_sf)
        if combine:
            y_bits = rows.recv_x.view(torch.int16).cpu().numpy().view(np.uint16)
            got = out_d.view(torch.int16).cpu().numpy().view(np.uint16)
            H.assert_combine_close(got, y_bits, wts, ref.expert_slot)
