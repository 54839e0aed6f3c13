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
# call on small batches, where it is one kernel. Then a small batch over 256
# experts at alignment 128, whose pad rows the scatter maps to row blocks and
# the one kernel deals out in chunks, and the combined call on several tiles:
# the one-launch layout, whose tiles exchange their counts through the
# workspace (every replay must leave the exchange words zero for the next),
# with its read-ahead, then the scatter.
@pytest.mark.parametrize("dtype,with_sf,alignment,t,combined,experts", [
    ("bf16", False, 1, 1500, False, 64), ("fp8", True, 16, 1500, False, 64),
    ("bf16", False, 1, 200, True, 64), ("fp8", True, 16, 256, True, 64),
    ("fp8", True, 128, 16, False, 256), ("fp8", True, 128, 16, True, 256),
    ("bf16", False, 1, 1500, True, 64), ("fp8", True, 16, 1500, True, 64)])
def test_captured_dispatch_replays_match_oracle(dtype, with_sf, alignment, t, combined, experts):
    print(f"\n[gpu-graph] capture dtype={dtype} sf={with_sf} A={alignment} T={t} combined={combined} E={experts}",
          flush=True)
    base = W.Workload("graph", t, 512, dtype, with_sf, experts, 8, 8, mask_frac=0.05, alignment=alignment, seed=31)
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
        assert M.dispatch_kernel_count(prob)[1] == (1 if t * k <= 2048 else 2)

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
        run = H.DeviceRun(prob, lay, rows, x_d, sf_d, ws)
        H.assert_layout_equal(run, ref)
        H.assert_rows_full(run, ref, inp.x_bytes(), inp.x_sf)
        if combine:
            y_bits = rows.recv_x.view(torch.int16).cpu().numpy().view(np.uint16)
            got = out_d.view(torch.int16).cpu().numpy().view(np.uint16)
            H.assert_combine_close(got, y_bits, wts, ref.expert_slot)


# The receiver-side expand captured the same way: its layout and scatter calls
# on a receive buffer of several tiles, and the one call on a small buffer.
@pytest.mark.parametrize("s_count,t,alignment,combined", [(4, 300, 16, False), (2, 40, 128, True)])
def test_captured_expand_replays_match_oracle(s_count, t, alignment, combined):
    from tests.test_gpu_expand import _compare, _receive_buffer, _source

    print(f"\n[gpu-graph] expand capture S={s_count} T={t} A={alignment} combined={combined}", flush=True)
    e, r, k, rank = 256, 8, 8, 3
    seeds = (201, 202, 203, 202)
    drawn = []
    for sd in seeds:
        sources = [_source(10 * sd + s, t, 512, "fp8", True, e, r, k, 0.05) for s in range(s_count)]
        drawn.append(_receive_buffer(sources, e, r, rank, slack=0, seed=sd))
    m = max(d[4] for d in drawn) + 3  # one stride for every replay
    row_bytes, sfw = drawn[0][1].shape[1], drawn[0][2].shape[1]

    def restride(d, seed):
        """The same received rows at stride m, junk in every unused row."""
        topk_i, buf_i, sf_i, counts, m_i = d
        rng = np.random.default_rng([seed, 57])
        topk = rng.integers(-3, e + 5, size=(s_count * m, k)).astype(np.int64)
        buf = rng.integers(0, 256, size=(s_count * m, row_bytes), dtype=np.uint8)
        sf = rng.uniform(-9, 9, size=(s_count * m, sfw)).astype(np.float32)
        for s in range(s_count):
            n = counts[s]
            topk[s * m:s * m + n] = topk_i[s * m_i:s * m_i + n]
            buf[s * m:s * m + n] = buf_i[s * m_i:s * m_i + n]
            sf[s * m:s * m + n] = sf_i[s * m_i:s * m_i + n]
        return topk, buf, sf, counts

    q = M.make_expand_problem(s_count, m, k, e, r, rank, alignment, 8, row_bytes, sfw)
    lay = M.alloc_expand_layout(q, H.DEVICE)
    ws = M.alloc_expand_workspace(q, H.DEVICE)
    cap = max(q.recv_capacity_rows, 1)
    recv_x = torch.empty((cap, row_bytes), dtype=torch.uint8, device=H.DEVICE)
    recv_sf = torch.empty((cap, sfw), dtype=torch.float32, device=H.DEVICE)
    topk_d = torch.zeros((s_count * m, k), dtype=torch.int64, device=H.DEVICE)
    counts_d = torch.zeros(s_count, dtype=torch.int32, device=H.DEVICE)
    buf_d = torch.zeros((s_count * m, row_bytes), dtype=torch.uint8, device=H.DEVICE)
    sf_d = torch.zeros((s_count * m, sfw), dtype=torch.float32, device=H.DEVICE)

    def load(i):
        topk, buf, sf, counts = restride(drawn[i], seeds[i])
        topk_d.copy_(torch.from_numpy(topk))
        counts_d.copy_(torch.from_numpy(counts.astype(np.int32)))
        buf_d.copy_(torch.from_numpy(buf))
        sf_d.copy_(torch.from_numpy(sf))
        for f in dataclasses.fields(lay):
            getattr(lay, f.name).fill_(H.CANARY)
        recv_x.fill_(H.ROW_FILL)
        recv_sf.view(torch.uint8).fill_(H.ROW_FILL)
        return topk, buf, sf, counts

    def step():
        if combined:
            M.dispatch_expand_layout_and_scatter(q, topk_d, counts_d, lay, ws, buf_d, sf_d, recv_x, recv_sf)
        else:
            M.dispatch_expand_layout(q, topk_d, counts_d, lay, ws)
            M.dispatch_expand_scatter(q, lay, buf_d, sf_d, recv_x, recv_sf)

    side = torch.cuda.Stream(device=H.DEVICE)
    load(0)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream, outside the graph
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()

    for i in range(1, len(seeds)):
        topk, buf, sf, counts = load(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.expand_layout(topk, counts, s_count, m, e, r, rank, alignment)
        assert ref.status == 0
        _compare(lay, recv_x, recv_sf, ref, buf, sf)
