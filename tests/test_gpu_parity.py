"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for bit.

Every count, psum, slot, inverse-map entry, status bit and copied byte must
equal the oracle's. Canary bands check that nothing past the totals is
written. Runs on an MI355X only (marked ``gpu``).
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
    print(f"\n[gpu-parity] {msg}", flush=True)


def _reduced(w: W.Workload, t: int) -> W.Workload:
    return dataclasses.replace(w, name=f"{w.name}_T{t}", num_tokens=t)


def _check_full(w: W.Workload, topk_bytes: int = 8):
    inp = W.make_inputs(w)
    xb = inp.x_bytes()
    ref = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment)
    run = H.run_gpu(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, xb, inp.x_sf,
                    topk_bytes=topk_bytes)
    H.assert_layout_equal(run, ref)
    H.assert_rows_full(run, ref, xb, inp.x_sf)


# Reduced-size variants of the five workloads: full element-by-element parity
# on every output, several tiles and a ragged last tile.
@pytest.mark.parametrize("name,t", [("tiny", 256), ("dsv3_bf16", 2500), ("dsv3_fp8_a128", 2311),
                                    ("zipf_bf16", 3001), ("ranklocal_fp8_a128", 2777)])
def test_reduced_workload_full_parity(name, t):
    w = _reduced(W.get(name), t)
    _banner(w.describe())
    _check_full(w)


# The five workloads at full size, in the launch configuration the benchmark
# times: the whole layout bit-exact, rows checked against the oracle on
# samples (full rows for the smaller ones) and on every row by a device gather.
# The benchmark times the combined call (the layout kernels read the token
# rows ahead for the scatter when they fit the Infinity Cache, and the
# scatter then bounds its workgroups per CU); the two separate calls are
# checked as well, plain and as the read-ahead layout plus the hinted scatter.
@pytest.mark.parametrize("combined,read_ahead", [(True, False), (False, False), (False, True)],
                         ids=["one_call", "two_calls", "two_calls_read_ahead"])
@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_workload_full_size(name, combined, read_ahead):
    w = W.get(name)
    _banner(f"{w.describe()} combined={combined} read_ahead={read_ahead}")
    inp = W.make_inputs(w)
    xb = inp.x_bytes()
    ref = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment)
    run = H.run_gpu(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, xb, inp.x_sf, combined=combined,
                    read_ahead=read_ahead)
    H.assert_layout_equal(run, ref)
    if w.num_tokens * w.row_bytes <= 64 << 20:
        H.assert_rows_full(run, ref, xb, inp.x_sf)
    else:
        H.assert_rows_sampled(run, ref, xb, inp.x_sf)
    H.assert_rows_gather_property(run, ref)


def _edge(topk, e, r, a, row_bytes=64, s=0, seed=0, **kw):
    t = topk.shape[0]
    xb = H.random_rows(seed, t, row_bytes)
    sf = None if s == 0 else np.random.default_rng([seed, 7]).uniform(0.5, 2, (t, s)).astype(np.float32)
    ref = oracle.layout(topk, e, r, a, recv_capacity=kw.get("recv_capacity"),
                        rank_capacity=kw.get("rank_capacity"))
    run = H.run_gpu(topk, e, r, a, xb, sf, **kw)
    H.assert_layout_equal(run, ref)
    if ref.status == 0:
        H.assert_rows_full(run, ref, xb, sf)
    return run, ref


def _uniform(seed, t, k, e, mask=0.0):
    w = W.Workload("edge", t, 64, "bf16", False, e, 1, k, mask_frac=mask, seed=seed)
    return W.make_topk(w)


# Up to 256 tokens at top-8 one workgroup lays the batch out in one launch
# (1 or 2 chunks per wavefront); from 257 on, tiles and two launches.
@pytest.mark.parametrize("t", [0, 1, 2, 63, 64, 65, 128, 129, 200, 256, 257, 1023, 1024, 1025])
def test_token_counts_around_tiles(t):
    _banner(f"T={t}")
    _edge(_uniform(3, t, 8, 256, 0.05), 256, 8, 4)


# Shapes on both sides of every layout geometry switch. While the tile
# histograms (16-wavefront tiles, 1/2/4/8 chunks per wavefront) hold at most
# 65536 ints, two launches; beyond, a column scan over 4-wavefront tiles.
# Very wide key sets narrow the tiles to what LDS holds. The combined call on
# the same shapes reads the rows ahead, and then lays out in one launch where
# the tiles can exchange their counts (up to 256 tiles of fewer than 4096
# (token, k) pairs whose exchange words fit the workspace's 8192-word
# region, a thread per count word); the comments name the combined call's
# layout.
@pytest.mark.parametrize("t,k,e,r", [
    (31744, 8, 256, 8),     # two launches, 1 chunk per wavefront, 248 tiles (the largest)
    (31745, 8, 256, 8),     # one launch, 2 chunks, 125 tiles
    (63489, 8, 256, 8),     # two launches, 4 chunks (4096 pairs per tile: past 12-bit exchange counts)
    (126977, 8, 256, 8),    # two launches, 8 chunks
    (253952, 8, 256, 8),    # two launches, 8 chunks, 248 tiles
    (253953, 8, 256, 8),    # column scan, 8 chunks per wavefront
    (768, 8, 4096, 1024),   # two launches, 5-wavefront tiles of 2 chunks (1025 words per tile)
    (3840, 8, 4096, 1024),  # two launches, 5-wavefront tiles of 8 chunks, 12 tiles (the largest)
    (3841, 8, 4096, 1024),  # column scan, 1 chunk
    (20000, 8, 4096, 1024), # column scan, 2 chunks
    (40000, 8, 4096, 1024), # column scan, 4 chunks
    (6000, 8, 2048, 1024),  # two launches, 11-wavefront tiles of 4 chunks (18 x 615 exchange words: past the region)
    (769, 8, 4096, 64),     # two launches, 7-wavefront tiles (833 words per tile)
    (70000, 2, 512, 16),    # one launch, top-2: 32 tokens per chunk
])
def test_layout_geometry_paths(t, k, e, r):
    _banner(f"geometry T={t} K={k} E={e} R={r}")
    _edge(_uniform(11, t, k, e, 0.05), e, r, 2, row_bytes=16)
    # The combined call on the same shape: its layout kernels carry the
    # read-ahead workgroups (and on the column-scan path, three kernels).
    _edge(_uniform(11, t, k, e, 0.05), e, r, 2, row_bytes=16, s=3, combined=True)


@pytest.mark.parametrize("k,e,r", [(1, 8, 2), (2, 16, 16), (3, 12, 4), (6, 64, 8), (7, 128, 128),
                                   (16, 64, 4), (32, 64, 8), (32, 32, 32), (5, 4096, 64), (8, 4096, 1024)])
def test_topk_and_expert_shapes(k, e, r):
    _banner(f"K={k} E={e} R={r}")
    _edge(_uniform(5, 777, k, e, 0.1), e, r, 3, row_bytes=48)


@pytest.mark.parametrize("a", [1, 2, 3, 64, 128, 1000])
def test_alignments(a):
    _banner(f"A={a}")
    _edge(_uniform(6, 900, 8, 64, 0.02), 64, 8, a, row_bytes=80, s=5)
    # Combined call: pad entries of the inverse map are dealt over the layout
    # workgroups only, not over the read-ahead workgroups of the same launch.
    _edge(_uniform(6, 900, 8, 64, 0.02), 64, 8, a, row_bytes=80, s=5, combined=True)


# Pad rows of small batches. While the routed rows can reach fewer blocks of
# A rows than there are experts (min(E, T*K) + T*K // A < E), the scatter maps
# its pad wavefronts to row blocks and finds each block's expert by a search
# over the psums (64 samples, then one chunk); otherwise one set of
# wavefronts per expert. Both sides of the switch, search chunks of 1, 2 and
# 64 experts, and scale factors in the pad rows.
@pytest.mark.parametrize("t,k,e,r,a", [
    (1, 8, 256, 8, 128),     # per block: 8 blocks of 256 experts
    (16, 8, 256, 8, 128),    # per block
    (31, 8, 256, 8, 128),    # per block: 249 blocks, the largest below 256
    (32, 8, 256, 8, 128),    # per expert: 258 blocks
    (3, 2, 65, 5, 7),        # per block, search chunks of 2 experts
    (40, 1, 64, 8, 2),       # per block, search chunks of 1 expert
    (100, 8, 4096, 8, 128),  # per block, search chunks of 64 experts
    (200, 8, 4096, 64, 3),   # per block, many partly filled blocks
    (511, 8, 4096, 8, 2),    # per expert: 6132 blocks
    (5, 1, 1, 1, 4),         # one expert: per expert
])
def test_pad_rows_of_small_batches(t, k, e, r, a):
    _banner(f"pads T={t} K={k} E={e} A={a}")
    _edge(_uniform(15, t, k, e, 0.1), e, r, a, row_bytes=80, s=3, seed=t)


def test_pad_rows_of_a_small_batch_at_exact_capacity():
    topk = _uniform(16, 12, 8, 256, 0.05)
    full = oracle.layout(topk, 256, 8, 128)
    _edge(topk, 256, 8, 128, row_bytes=80, s=3, recv_capacity=full.num_recv_rows)
    run, ref = _edge(topk, 256, 8, 128, row_bytes=80, s=3, recv_capacity=full.num_recv_rows - 1)
    assert ref.status == oracle.RECV_OVERFLOW
    assert np.all(run.rows.recv_x.cpu().numpy() == H.ROW_FILL)


def test_fully_masked_tokens():
    topk = _uniform(7, 500, 4, 32)
    topk[::3] = -1
    topk[1::7, :2] = -5  # any negative value is masked
    _edge(topk, 32, 4, 8)


def test_all_tokens_on_few_experts():
    w = W.Workload("single", 3000, 64, "bf16", False, 128, 16, 8, routing=W.ROUTING_SINGLE)
    _edge(W.make_topk(w), 128, 16, 64)


def test_one_expert_per_rank_and_one_rank():
    _edge(_uniform(8, 1500, 8, 64), 64, 64, 1)
    _edge(_uniform(9, 1500, 8, 64), 64, 1, 2)


def test_int32_routing_table():
    w = _reduced(W.get("dsv3_bf16"), 1800)
    _banner("int32 topk")
    _check_full(w, topk_bytes=4)


@pytest.mark.parametrize("row_bytes,s", [(16, 1), (208, 3), (1040, 70), (32768, 0), (40976, 130)])
def test_row_and_scale_factor_widths(row_bytes, s):
    _banner(f"row_bytes={row_bytes} S={s}")
    _edge(_uniform(10, 300, 4, 32, 0.1), 32, 4, 4, row_bytes=row_bytes, s=s)


@pytest.mark.parametrize("flags", [1, 2, 3, 6, 7])
def test_output_selection(flags):
    _banner(f"flags={flags}")
    _edge(_uniform(11, 400, 8, 64, 0.05), 64, 8, 16, row_bytes=96, s=2, flags=flags)


def test_status_bad_expert_writes_nothing():
    topk = _uniform(12, 300, 4, 16)
    topk[123, 2] = 16
    run, ref = _edge(topk, 16, 4, 1)
    assert ref.status == oracle.BAD_EXPERT
    assert np.all(run.layout.expert_slot.cpu().numpy() == H.CANARY)
    for name in ("rank_x", "recv_x"):
        assert np.all(getattr(run.rows, name).cpu().numpy() == H.ROW_FILL)


def test_status_duplicate_expert():
    topk = _uniform(13, 300, 4, 16)
    topk[77, 3] = topk[77, 0]
    run, ref = _edge(topk, 16, 4, 2)
    assert ref.status == oracle.DUP_EXPERT


def test_status_capacity_overflow_writes_nothing():
    topk = _uniform(14, 600, 8, 64)
    mr, mk = oracle.max_rows(600, 8, 64, 8, 4)
    full = oracle.layout(topk, 64, 8, 4)
    run, ref = _edge(topk, 64, 8, 4, recv_capacity=full.num_recv_rows - 1, rank_capacity=mk)
    assert ref.status == oracle.RECV_OVERFLOW
    assert np.all(run.rows.recv_x.cpu().numpy() == H.ROW_FILL)
    run, ref = _edge(topk, 64, 8, 4, recv_capacity=mr, rank_capacity=full.num_rank_rows - 1)
    assert ref.status == oracle.RANK_OVERFLOW
    assert np.all(run.rows.rank_x.cpu().numpy() == H.ROW_FILL)
    _edge(topk, 64, 8, 4, recv_capacity=full.num_recv_rows, rank_capacity=full.num_rank_rows)


def test_deterministic_repeats_and_workspace_reuse():
    """Ten runs give identical bits; one workspace serves calls of different sizes."""
    w = W.get("dsv3_bf16")
    inp = W.make_inputs(w)
    xb = inp.x_bytes()
    ref = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment)
    first = H.run_gpu(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, xb)
    H.assert_layout_equal(first, ref)
    ws = first.workspace
    for i in range(10):
        run = H.run_gpu(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, xb, workspace=ws)
        for f in dataclasses.fields(run.layout):
            assert torch.equal(getattr(run.layout, f.name), getattr(first.layout, f.name)), (i, f.name)
        assert torch.equal(run.rows.recv_x, first.rows.recv_x) and torch.equal(run.rows.rank_x, first.rows.rank_x)
    small = _uniform(15, 333, 8, 256, 0.05)
    ref_s = oracle.layout(small, 256, 8, 1)
    run_s = H.run_gpu(small, 256, 8, 1, H.random_rows(1, 333, 64), workspace=ws)
    H.assert_layout_equal(run_s, ref_s)
    run = H.run_gpu(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, xb, workspace=ws)
    H.assert_layout_equal(run, ref)


def test_replay_scatter_with_saved_layout():
    """Cached dispatch: the layout is computed once and reused to scatter new
    token batches with the same routing (the page's cached mode, sections 6.2
    and 8.3); every replay matches the oracle and leaves the layout untouched."""
    w = _reduced(W.get("dsv3_fp8_a128"), 1500)
    _banner("replay " + w.describe())
    inp = W.make_inputs(w)
    ref = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment)
    run = H.run_gpu(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, inp.x_bytes(), inp.x_sf)
    H.assert_layout_equal(run, ref)
    saved = {f.name: getattr(run.layout, f.name).clone() for f in dataclasses.fields(run.layout)}
    import moe_token_dispatch_amd as M

    for seed in (101, 102):
        xb = H.random_rows(seed, w.num_tokens, w.row_bytes)
        sf = np.random.default_rng([seed, 5]).uniform(0.5, 2, (w.num_tokens, w.sf_per_token)).astype(np.float32)
        x_d = torch.from_numpy(xb).to(H.DEVICE)
        sf_d = torch.from_numpy(sf).to(H.DEVICE)
        M.dispatch_scatter(run.problem, run.layout, x_d, sf_d, run.rows.rank_x, run.rows.rank_sf,
                           run.rows.recv_x, run.rows.recv_sf)
        torch.cuda.synchronize()
        run.x, run.x_sf = x_d, sf_d
        want = oracle.scatter(ref, xb, sf)
        p_total, n_rank = ref.num_recv_rows, ref.num_rank_rows
        assert np.array_equal(run.rows.recv_x[:p_total].cpu().numpy(), want.recv_x), seed
        assert np.array_equal(run.rows.rank_x[:n_rank].cpu().numpy(), want.rank_x), seed
        assert np.array_equal(run.rows.recv_sf[:p_total].cpu().numpy().view(np.int32), want.recv_sf.view(np.int32))
        assert np.array_equal(run.rows.rank_sf[:n_rank].cpu().numpy().view(np.int32), want.rank_sf.view(np.int32))
        for name, t in saved.items():
            assert torch.equal(getattr(run.layout, name), t), f"scatter changed layout field {name}"


def test_expert_count_cumulative_adds_successful_calls():
    """The optional running per-expert totals: each call that ends with status 0
    adds its expert_count (before alignment); a failed call adds nothing."""
    _banner("expert_count_cumulative")
    e, r, k, t, a = 64, 8, 6, 700, 4
    prob = M.make_problem(t, k, e, r, a, 8, 16, 0)
    lay, ws = M.alloc_layout(prob, H.DEVICE), M.alloc_workspace(prob, H.DEVICE)
    start = (np.arange(e, dtype=np.int64) * 3 - 50).astype(np.int32)  # any values the caller holds
    cum = torch.from_numpy(start).to(H.DEVICE)
    want = start.astype(np.int64)
    for seed in (41, 42, 43):
        topk = _uniform(seed, t, k, e, 0.1)
        M.dispatch_layout(prob, torch.from_numpy(topk).to(H.DEVICE), lay, ws, expert_count_cumulative=cum)
        want += oracle.layout(topk, e, r, a).expert_count
    bad = _uniform(44, t, k, e)
    bad[5, 1] = e
    M.dispatch_layout(prob, torch.from_numpy(bad).to(H.DEVICE), lay, ws, expert_count_cumulative=cum)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == oracle.BAD_EXPERT
    assert np.array_equal(cum.cpu().numpy(), want)
    # Through a prepared plan as well: one more successful call.
    topk = _uniform(45, t, k, e, 0.1)
    plan = M.Plan(prob, torch.from_numpy(topk).to(H.DEVICE), lay, ws, expert_count_cumulative=cum)
    plan.layout()
    torch.cuda.synchronize()
    assert np.array_equal(cum.cpu().numpy(), want + oracle.layout(topk, e, r, a).expert_count)
    with pytest.raises(ValueError):
        M.dispatch_layout(prob, torch.from_numpy(topk).to(H.DEVICE), lay, ws,
                          expert_count_cumulative=cum[:e - 1])
