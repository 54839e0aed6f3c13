"""Broad seeded sweeps of small and mid-sized problems against the CPU oracle:
the dispatch and the receiver-side expand bit for bit through both call
forms, and the combine within its bound.

Each seed draws every parameter at once (tokens across the tile, chunk,
one-kernel and pad-mapping boundaries; top-k; experts and ranks; alignment;
routing width; masking; output selection; row and scale-factor widths) with
narrow rows, so that a few hundred problems run in seconds. Every problem is
printed before it runs.
"""

import numpy as np
import pytest
import torch

import moe_token_dispatch_amd as M
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

BATCHES = 8
PER_BATCH = 100


def _draw(seed):
    rng = np.random.default_rng([seed, 9090])
    r = int(rng.choice([1, 2, 3, 4, 8, 16, 64, 256, 1024]))
    epr = int(rng.choice([1, 1, 2, 4, 8, 16, 32]))
    e = min(r * epr, 4096) // r * r
    k = int(min(e, rng.choice([1, 2, 3, 4, 5, 8, 8, 12, 16, 32])))
    t = int(rng.choice([0, 1, 2, 3, 8, 15, 31, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 300, 384, 385,
                        511, 512, 513, 777, 1023, 1024, 1025, 1500, 2047, 2500]))
    a = int(rng.choice([1, 1, 2, 3, 7, 64, 128]))
    row_bytes = int(rng.choice([16, 32, 48, 64, 1040]))
    s = int(rng.choice([0, 0, 1, 2, 5]))
    topk_bytes = int(rng.choice([4, 8]))
    mask = float(rng.choice([0.0, 0.0, 0.03, 0.3, 1.0]))
    flags = int(rng.choice([M.ALL_OUTPUTS, M.ALL_OUTPUTS, M.EXPERT_MAJOR | M.ZERO_PAD, M.EXPERT_MAJOR,
                            M.RANK_CONTIG, M.RANK_CONTIG | M.EXPERT_MAJOR]))
    combined = bool(rng.integers(0, 2))
    if (t * k + e * (a - 1)) * (row_bytes + 4 * s) > 64 << 20:  # keep every case quick to check
        row_bytes, s = 16, 0
    return t, k, e, r, a, row_bytes, s, topk_bytes, mask, flags, combined


@pytest.mark.parametrize("batch", range(BATCHES))
def test_seeded_sweep(batch):
    for seed in range(batch * PER_BATCH, (batch + 1) * PER_BATCH):
        t, k, e, r, a, row_bytes, s, topk_bytes, mask, flags, combined = _draw(seed)
        print(f"[gpu-sweep] seed={seed} T={t} K={k} E={e} R={r} A={a} row={row_bytes} S={s} idx={topk_bytes} "
              f"mask={mask} flags={flags} one_call={combined}", flush=True)
        w = W.Workload(f"sweep{seed}", t, 64, "bf16", False, e, r, k, mask_frac=mask, seed=5000 + seed)
        topk = W.make_topk(w)
        xb = H.random_rows(seed, t, row_bytes)
        sf = None if s == 0 else np.random.default_rng([seed, 11]).uniform(0.5, 2, (t, s)).astype(np.float32)
        ref = oracle.layout(topk, e, r, a)
        assert ref.status == 0
        run = H.run_gpu(topk, e, r, a, xb, sf, topk_bytes=topk_bytes, flags=flags, combined=combined)
        H.assert_layout_equal(run, ref)
        H.assert_rows_full(run, ref, xb, sf)


EXPAND_BATCHES = 4
EXPAND_PER_BATCH = 50


def _draw_expand(seed):
    rng = np.random.default_rng([seed, 9191])
    r = int(rng.choice([1, 2, 4, 8, 16, 64]))
    e = r * int(rng.choice([1, 2, 4, 8, 32]))
    k = int(min(e, rng.choice([1, 2, 3, 4, 8, 9])))
    s_count = int(rng.choice([1, 2, 3, 5, 8]))
    t = int(rng.choice([1, 3, 17, 64, 200, 600]))
    a = int(rng.choice([1, 1, 2, 3, 16, 128]))
    rank = int(rng.integers(0, r))
    hidden = int(rng.choice([64, 128, 512]))
    dtype = str(rng.choice(["bf16", "fp8"]))
    with_sf = dtype == "fp8" and hidden >= 128 and bool(rng.integers(0, 2))
    mask = float(rng.choice([0.0, 0.1, 0.5]))
    slack = int(rng.choice([0, 0, 5]))
    topk_bytes = int(rng.choice([4, 8]))
    combined = bool(rng.integers(0, 2))
    return s_count, t, hidden, dtype, with_sf, e, r, k, mask, rank, a, slack, topk_bytes, combined


@pytest.mark.parametrize("batch", range(EXPAND_BATCHES))
def test_seeded_expand_sweep(batch):
    from tests.test_gpu_expand import _compare, _receive_buffer, _run_expand, _source

    for seed in range(batch * EXPAND_PER_BATCH, (batch + 1) * EXPAND_PER_BATCH):
        s_count, t, hidden, dtype, with_sf, e, r, k, mask, rank, a, slack, ib, combined = _draw_expand(seed)
        print(f"[gpu-sweep] expand seed={seed} S={s_count} T={t} H={hidden} {dtype}{'+sf' if with_sf else ''} "
              f"E={e} R={r} K={k} rank={rank} A={a} slack={slack} idx={ib} one_call={combined}", flush=True)
        sources = [_source(70000 + 17 * seed + s, t, hidden, dtype, with_sf, e, r, k, mask) for s in range(s_count)]
        recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, slack=slack, seed=seed)
        ref = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a)
        assert ref.status == 0
        _, lay, recv_x, recv_sf_out = _run_expand(recv_topk, recv_buf, recv_sf, counts, m, e, r, rank, a,
                                                  topk_bytes=ib, combined=combined)
        _compare(lay, recv_x, recv_sf_out, ref, recv_buf, recv_sf)


COMBINE_BATCHES = 2
COMBINE_PER_BATCH = 50


def _draw_combine(seed):
    rng = np.random.default_rng([seed, 9292])
    t = int(rng.choice([1, 2, 31, 64, 65, 300, 1000]))
    e = int(rng.choice([8, 32, 64, 256]))
    k = int(min(e, rng.choice([1, 2, 3, 6, 8, 9, 16, 32])))
    hidden = 8 * int(rng.choice([1, 7, 16, 63, 64, 65, 128, 256]))
    mask = float(rng.choice([0.0, 0.05, 0.5, 1.0]))
    alignment = int(rng.choice([1, 1, 4, 16]))
    return t, k, e, hidden, mask, alignment


@pytest.mark.parametrize("batch", range(COMBINE_BATCHES))
def test_seeded_combine_sweep(batch):
    from tests.test_gpu_combine import _combine_inputs, _run_combine

    for seed in range(batch * COMBINE_PER_BATCH, (batch + 1) * COMBINE_PER_BATCH):
        t, k, e, hidden, mask, alignment = _draw_combine(seed)
        print(f"[gpu-sweep] combine seed={seed} T={t} K={k} E={e} H={hidden} mask={mask} A={alignment}", flush=True)
        w, topk, ref, y, wts = _combine_inputs(t, k, e, hidden, mask, seed=90000 + seed, alignment=alignment)
        got = _run_combine(ref.expert_slot, wts, y)
        H.assert_combine_close(got, y.view(torch.int16).numpy().view(np.uint16), wts, ref.expert_slot)
