"""GPU parity of the receiver-side expand (the page's copy epilogue) against the
CPU oracle, bit for bit, through the C ABI.

Receive buffers are assembled on the host from seeded source batches: source
s's rows for receiver r are its tokens routed to at least one of r's experts,
in token order, placed at rows [s*M, s*M + count) of a fixed-stride buffer;
the rest of every region holds junk that must never be read.
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


def _banner(msg):
    print(f"\n[gpu-expand] {msg}", flush=True)


def _source(seed, t, hidden, dtype, with_sf, e, r, k, mask):
    w = W.Workload(f"src{seed}", t, hidden, dtype, with_sf, e, r, k, mask_frac=mask, seed=seed)
    inp = W.make_inputs(w)
    return w, inp


def _receive_buffer(sources, e, r, rank, slack, seed):
    """Host-side plumbing: gather each source's rows for `rank` into a fixed-stride buffer."""
    epr = e // r
    picks = []
    for w, inp in sources:
        topk = inp.topk_idx
        mine = ((topk >= rank * epr) & (topk < (rank + 1) * epr)).any(axis=1)
        picks.append(np.nonzero(mine)[0])
    m = max(len(p) for p in picks) + slack
    s_count = len(sources)
    k = sources[0][1].topk_idx.shape[1]
    row_bytes = sources[0][0].row_bytes
    sfw = sources[0][0].sf_per_token
    rng = np.random.default_rng([seed, 31])
    recv_topk = rng.integers(-3, e + 5, size=(s_count * m, k)).astype(np.int64)  # junk
    recv_buf = rng.integers(0, 256, size=(s_count * m, row_bytes), dtype=np.uint8)
    recv_sf = rng.uniform(-9, 9, size=(s_count * m, sfw)).astype(np.float32) if sfw else None
    counts = np.zeros(s_count, dtype=np.int32)
    for s, ((w, inp), pick) in enumerate(zip(sources, picks)):
        n = len(pick)
        counts[s] = n
        recv_topk[s * m:s * m + n] = inp.topk_idx[pick]
        recv_buf[s * m:s * m + n] = inp.x_bytes()[pick]
        if sfw:
            recv_sf[s * m:s * m + n] = inp.x_sf[pick]
    return recv_topk, recv_buf, recv_sf, counts, m


def _run_expand(recv_topk, recv_buf, recv_sf, counts, m, e, r, rank, a, topk_bytes=8, capacity=None,
                combined=False):
    s_count, k = len(counts), recv_topk.shape[1]
    q = M.make_expand_problem(s_count, m, k, e, r, rank, a, topk_bytes, recv_buf.shape[1],
                              0 if recv_sf is None else recv_sf.shape[1], capacity)
    lay = M.alloc_expand_layout(q, H.DEVICE)
    for f in dataclasses.fields(lay):
        getattr(lay, f.name).fill_(H.CANARY)
    ws = M.alloc_expand_workspace(q, H.DEVICE)
    cap = max(q.recv_capacity_rows, 1)
    recv_x = torch.full((cap, recv_buf.shape[1]), H.ROW_FILL, dtype=torch.uint8, device=H.DEVICE)
    sfw = 0 if recv_sf is None else recv_sf.shape[1]
    recv_sf_out = None
    if sfw:
        recv_sf_out = torch.empty((cap, sfw), dtype=torch.float32, device=H.DEVICE)
        recv_sf_out.view(torch.uint8).fill_(H.ROW_FILL)
    dt = np.int64 if topk_bytes == 8 else np.int32
    topk_d = torch.from_numpy(recv_topk.astype(dt)).to(H.DEVICE)
    counts_d = torch.from_numpy(counts.astype(np.int32)).to(H.DEVICE)
    buf_d = torch.from_numpy(recv_buf).to(H.DEVICE)
    sf_d = None if recv_sf is None else torch.from_numpy(recv_sf).to(H.DEVICE)
    if combined:
        M.dispatch_expand_layout_and_scatter(q, topk_d, counts_d, lay, ws, buf_d, sf_d, recv_x, recv_sf_out)
    else:
        M.dispatch_expand_layout(q, topk_d, counts_d, lay, ws)
        M.dispatch_expand_scatter(q, lay, buf_d, sf_d, recv_x, recv_sf_out)
    torch.cuda.synchronize()
    return q, lay, recv_x, recv_sf_out


def _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf):
    assert int(lay.status.item()) == ref.status, (int(lay.status.item()), ref.status)
    assert np.array_equal(lay.expert_count.cpu().numpy(), ref.expert_count)
    assert np.array_equal(lay.expert_psum.cpu().numpy(), ref.expert_psum)
    if ref.status != 0:
        return
    p = ref.num_recv_rows
    assert np.array_equal(lay.expert_slot.cpu().numpy(), ref.expert_slot)
    src = lay.recv_src_row_idx.cpu().numpy()
    assert np.array_equal(src[:p], ref.recv_src_row_idx[:p])
    assert np.all(src[p:] == H.CANARY), "recv_src_row_idx written past the total"
    want = oracle.expand_scatter(ref, recv_buf, recv_sf, fill=H.ROW_FILL)
    got = recv_x.cpu().numpy()
    assert np.array_equal(got[:p], want.recv_x), "expert-major rows differ from the oracle"
    assert np.all(got[p:] == H.ROW_FILL), "rows written past the total"
    if recv_sf is not None:
        gs = recv_sf_out.view(torch.uint8).cpu().numpy()
        assert np.array_equal(gs[:p], want.recv_sf.view(np.uint8))
        assert np.all(gs[p:] == H.ROW_FILL)


@pytest.mark.parametrize("s_count,a,dtype,with_sf,rank", [
    (1, 1, "bf16", False, 0), (3, 1, "bf16", False, 5), (4, 128, "fp8", True, 2), (8, 16, "fp8", True, 7)])
def test_expand_multi_source(s_count, a, dtype, with_sf, rank):
    _banner(f"S={s_count} A={a} {dtype}{'+sf' if with_sf else ''} rank={rank}")
    e, r, k = 256, 8, 8
    sources = [_source(100 + s, 700 + 37 * s, 1024, dtype, with_sf, e, r, k, 0.05) for s in range(s_count)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, slack=13, seed=s_count)
    ref = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a)
    _, lay, recv_x, recv_sf_out = _run_expand(recv_topk, recv_buf, recv_sf, counts, m, e, r, rank, a)
    _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf)


def test_expand_int32_table_and_skewed_routing():
    e, r, k = 128, 16, 8
    sources = []
    for s in range(3):
        w = W.Workload(f"z{s}", 900, 512, "bf16", False, e, r, k, routing=W.ROUTING_ZIPF, mask_frac=0.02, seed=40 + s)
        sources.append((w, W.make_inputs(w)))
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, 3, slack=0, seed=9)
    ref = oracle.expand_layout(recv_topk, counts, 3, m, e, r, 3, 4)
    _, lay, recv_x, recv_sf_out = _run_expand(recv_topk, recv_buf, recv_sf, counts, m, e, r, 3, 4, topk_bytes=4)
    _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf)


def test_expand_end_to_end_single_source_matches_sender():
    """Device-only pipeline: the sender's rank-contiguous rows feed each
    receiver's expand; the receivers' expert-major buffers, side by side, are
    the sender's own expert-major buffer (one source), and every receiver
    matches the oracle."""
    w = dataclasses.replace(W.get("dsv3_fp8_a128"), num_tokens=1800)
    _banner("end-to-end " + w.describe())
    inp = W.make_inputs(w)
    xb = inp.x_bytes()
    e, r, a = w.num_experts, w.num_ranks, w.alignment
    send = H.run_gpu(inp.topk_idx, e, r, a, xb, inp.x_sf)
    ref_send = oracle.layout(inp.topk_idx, e, r, a)
    H.assert_layout_equal(send, ref_send)
    rank_psum = send.layout.rank_psum.cpu().numpy()
    rank_src = send.layout.rank_src_token_idx
    topk_d = torch.from_numpy(inp.topk_idx).to(H.DEVICE)
    epr = e // r
    for rank in range(r):
        lo, hi = int(rank_psum[rank]), int(rank_psum[rank + 1])
        m = hi - lo
        q = M.make_expand_problem(1, m, w.num_topk, e, r, rank, a, 8, w.row_bytes, w.sf_per_token)
        lay = M.alloc_expand_layout(q, H.DEVICE)
        ws = M.alloc_expand_workspace(q, H.DEVICE)
        cap = max(q.recv_capacity_rows, 1)
        recv_x = torch.empty((cap, w.row_bytes), dtype=torch.uint8, device=H.DEVICE)
        recv_sf = torch.empty((cap, w.sf_per_token), dtype=torch.float32, device=H.DEVICE)
        counts = torch.tensor([m], dtype=torch.int32, device=H.DEVICE)
        recv_topk = topk_d.index_select(0, rank_src[lo:hi].long()).contiguous()
        M.dispatch_expand_layout(q, recv_topk, counts, lay, ws)
        M.dispatch_expand_scatter(q, lay, send.rows.rank_x[lo:hi].contiguous(), send.rows.rank_sf[lo:hi].contiguous(),
                                  recv_x, recv_sf)
        torch.cuda.synchronize()
        assert int(lay.status.item()) == 0
        base = int(ref_send.expert_psum[rank * epr])
        p = int(lay.expert_psum[-1].item())
        assert p == int(ref_send.expert_psum[(rank + 1) * epr]) - base
        assert torch.equal(recv_x[:p], send.rows.recv_x[base:base + p]), rank
        assert torch.equal(recv_sf[:p].view(torch.int32), send.rows.recv_sf[base:base + p].view(torch.int32)), rank


def test_expand_status_bad_count_and_bad_expert():
    e, r, k = 32, 4, 4
    sources = [_source(60 + s, 200, 256, "bf16", False, e, r, k, 0.0) for s in range(2)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, 1, slack=3, seed=60)
    bad_counts = counts.copy()
    bad_counts[1] = m + 1
    ref = oracle.expand_layout(recv_topk, bad_counts, 2, m, e, r, 1, 1)
    # the overlong count also makes the region's unused junk rows live, whose
    # ids past E add the bad-expert bit; the GPU must report the same bits
    assert ref.status & oracle.BAD_COUNT
    _, lay, recv_x, _ = _run_expand(recv_topk, recv_buf, recv_sf, bad_counts, m, e, r, 1, 1)
    _compare(lay, recv_x, None, ref, recv_buf, recv_sf)
    assert np.all(recv_x.cpu().numpy() == H.ROW_FILL)
    bad = recv_topk.copy()
    bad[2, 1] = e
    ref = oracle.expand_layout(bad, counts, 2, m, e, r, 1, 1)
    assert ref.status == oracle.BAD_EXPERT
    _, lay, recv_x, _ = _run_expand(bad, recv_buf, recv_sf, counts, m, e, r, 1, 1)
    _compare(lay, recv_x, None, ref, recv_buf, recv_sf)


@pytest.mark.parametrize("m,counts", [(0, [0, 0]), (5, [0, 0]), (5, [5, 0])])
def test_expand_empty_and_partial(m, counts):
    e, r, k = 16, 2, 2
    rng = np.random.default_rng(5)
    recv_topk = rng.integers(0, e, size=(2 * m, k)).astype(np.int64)
    recv_topk[:, 1] = (recv_topk[:, 0] + 1) % e
    recv_buf = rng.integers(0, 256, size=(2 * m, 32), dtype=np.uint8)
    c = np.array(counts, dtype=np.int32)
    ref = oracle.expand_layout(recv_topk, c, 2, m, e, r, 0, 4)
    _, lay, recv_x, _ = _run_expand(recv_topk, recv_buf, None, c, m, e, r, 0, 4)
    _compare(lay, recv_x, None, ref, recv_buf, None)


# Receive buffers so small that their routed rows reach fewer blocks of A
# rows than the receiver has experts: the scatter maps its pad wavefronts to
# row blocks (the assert below checks that the case is one).
@pytest.mark.parametrize("s_count,t,a,rank", [(1, 3, 128, 3), (2, 1, 128, 0), (2, 1, 3, 6)])
def test_expand_pads_of_a_small_receive_buffer(s_count, t, a, rank):
    _banner(f"small receive buffer S={s_count} T={t} A={a} rank={rank}")
    e, r, k = 256, 8, 8
    sources = [_source(900 + 7 * s + t, t, 512, "fp8", True, e, r, k, 0.0) for s in range(s_count)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, slack=0, seed=t)
    pairs = s_count * m * k
    assert counts.sum() > 0 and min(pairs, e // r) + pairs // a < e // r
    ref = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a)
    _, lay, recv_x, recv_sf_out = _run_expand(recv_topk, recv_buf, recv_sf, counts, m, e, r, rank, a)
    _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf)


def _draw_expand(seed):
    rng = np.random.default_rng([seed, 77])
    r = int(rng.choice([1, 2, 4, 8, 16]))
    e = r * int(rng.choice([1, 2, 8, 32]))
    k = int(min(e, rng.choice([1, 2, 4, 8, 9])))
    s_count = int(rng.choice([1, 2, 5, 8]))
    t = int(rng.choice([1, 30, 300, 1500]))
    a = int(rng.choice([1, 1, 3, 16, 128]))
    rank = int(rng.integers(0, r))
    hidden = int(rng.choice([64, 512, 2048]))
    dtype = str(rng.choice(["bf16", "fp8"]))
    with_sf = dtype == "fp8" and bool(rng.integers(0, 2)) and hidden >= 128
    mask = float(rng.choice([0.0, 0.1]))
    slack = int(rng.choice([0, 7]))
    topk_bytes = int(rng.choice([4, 8]))
    return s_count, t, hidden, dtype, with_sf, e, r, k, mask, rank, a, slack, topk_bytes


@pytest.mark.parametrize("seed", range(12))
def test_expand_random_problem(seed):
    """Seeded random receivers (sources, rows, top-k, experts, ranks, this
    rank, alignment, row width, scale factors, slack, table width), each
    bit-exact against the oracle."""
    s_count, t, hidden, dtype, with_sf, e, r, k, mask, rank, a, slack, ib = _draw_expand(seed)
    _banner(f"random seed={seed} S={s_count} T={t} H={hidden} {dtype}{'+sf' if with_sf else ''} E={e} R={r} "
            f"K={k} rank={rank} A={a} slack={slack} idx={ib}")
    sources = [_source(5000 + 31 * seed + s, t, hidden, dtype, with_sf, e, r, k, mask) for s in range(s_count)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, slack=slack, seed=seed)
    ref = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a)
    assert ref.status == 0
    _, lay, recv_x, recv_sf_out = _run_expand(recv_topk, recv_buf, recv_sf, counts, m, e, r, rank, a, topk_bytes=ib)
    _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf)


def test_expand_expert_count_cumulative():
    """Running totals of the local experts' received rows over calls."""
    _banner("expand expert_count_cumulative")
    e, r, k, rank, a = 64, 4, 8, 2, 2
    sources = [_source(60 + s, 300, 64, "bf16", False, e, r, k, 0.05) for s in range(3)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, 5, 61)
    q = M.make_expand_problem(3, m, k, e, r, rank, a, 8, recv_buf.shape[1], 0)
    lay, ws = M.alloc_expand_layout(q, H.DEVICE), M.alloc_expand_workspace(q, H.DEVICE)
    ref = oracle.expand_layout(recv_topk, counts, 3, m, e, r, rank, a)
    assert ref.status == 0
    cum = torch.full((e // r,), 5, dtype=torch.int32, device=H.DEVICE)
    topk_d, counts_d = torch.from_numpy(recv_topk).to(H.DEVICE), torch.from_numpy(counts).to(H.DEVICE)
    for _ in range(2):
        M.dispatch_expand_layout(q, topk_d, counts_d, lay, ws, expert_count_cumulative=cum)
    torch.cuda.synchronize()
    assert np.array_equal(cum.cpu().numpy(), 5 + 2 * ref.expert_count.astype(np.int64))


# dispatch_expand_layout_and_scatter: one kernel for a small receive buffer
# (S * M * K up to 2048 entries), else the layout and scatter kernels.
@pytest.mark.parametrize("s_count,t,a,dtype,with_sf,rank", [
    (8, 28, 1, "bf16", False, 3),    # 8 x 31 rows x top-8 = 1984 entries: one kernel
    (8, 30, 1, "bf16", False, 3),    # 8 x 33 rows x top-8 = 2112 entries: the layout and scatter kernels
    (3, 80, 16, "fp8", True, 1),     # 1848 entries: one kernel, pads and scale factors
    (1, 250, 4, "bf16", False, 0),   # 1800 entries: one kernel
    (4, 300, 2, "fp8", True, 2),     # 8800 entries: the layout and scatter kernels
])
def test_expand_layout_and_scatter_in_one_call(s_count, t, a, dtype, with_sf, rank):
    _banner(f"one call: S={s_count} T={t} A={a} {dtype} sf={with_sf} rank={rank}")
    e, r, k = 64, 4, 8
    sources = [_source(70 + i, t, 128, dtype, with_sf, e, r, k, 0.05) for i in range(s_count)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, 3, 71)
    ref = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a)
    q, lay, recv_x, recv_sf_out = _run_expand(recv_topk, recv_buf, recv_sf, counts, m, e, r, rank, a,
                                              combined=True)
    _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf)


def test_expand_one_call_bad_count_writes_nothing():
    _banner("one call: bad count")
    e, r, k = 32, 4, 4
    sources = [_source(80 + i, 60, 64, "bf16", False, e, r, k, 0.0) for i in range(2)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, 1, 2, 81)
    bad = counts.copy()
    bad[1] = m + 1
    ref = oracle.expand_layout(recv_topk, bad, 2, m, e, r, 1, 1)
    # The count past M flags BAD_COUNT (and, through the junk rows it then
    # covers, possibly BAD_EXPERT too); either way nothing is written.
    assert ref.status & oracle.BAD_COUNT
    q, lay, recv_x, _ = _run_expand(recv_topk, recv_buf, None, bad, m, e, r, 1, 1, combined=True)
    _compare(lay, recv_x, None, ref, recv_buf, None)
    assert np.all(recv_x.cpu().numpy() == H.ROW_FILL)


def test_expand_plan_layout_scatter_and_one_call():
    """The prepared expand: two calls, then the one call, both equal the oracle."""
    _banner("expand plan")
    e, r, k, rank, a = 64, 4, 8, 2, 4
    sources = [_source(90 + i, 120, 128, "fp8", True, e, r, k, 0.05) for i in range(3)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, 2, 91)
    ref = oracle.expand_layout(recv_topk, counts, 3, m, e, r, rank, a)
    q = M.make_expand_problem(3, m, k, e, r, rank, a, 8, recv_buf.shape[1], recv_sf.shape[1])
    lay, ws = M.alloc_expand_layout(q, H.DEVICE), M.alloc_expand_workspace(q, H.DEVICE)
    cap = max(q.recv_capacity_rows, 1)
    for one_call in (False, True):
        for f in dataclasses.fields(lay):
            getattr(lay, f.name).fill_(H.CANARY)
        recv_x = torch.full((cap, recv_buf.shape[1]), H.ROW_FILL, dtype=torch.uint8, device=H.DEVICE)
        recv_sf_out = torch.empty((cap, recv_sf.shape[1]), dtype=torch.float32, device=H.DEVICE)
        recv_sf_out.view(torch.uint8).fill_(H.ROW_FILL)
        plan = M.ExpandPlan(q, torch.from_numpy(recv_topk).to(H.DEVICE), torch.from_numpy(counts).to(H.DEVICE), lay,
                            ws, torch.from_numpy(recv_buf).to(H.DEVICE), torch.from_numpy(recv_sf).to(H.DEVICE),
                            recv_x, recv_sf_out)
        if one_call:
            plan()
        else:
            plan.layout()
            plan.scatter()
        torch.cuda.synchronize()
        _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf)
