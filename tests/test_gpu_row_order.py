"""The destination-ordered scatter (layouts that carry a row order, rows of
4 KB or more) and the source-major scatter (no row order), each bit for bit
against the CPU oracle on the same inputs, and the row order itself against
the oracle's inverse maps (every routed row once, in runs of consecutive
tokens, grouped by key in slot order; checked in assert_layout_equal)."""

import numpy as np
import pytest

import moe_token_dispatch_amd as M
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _topk(seed, t, k, e, mask):
    w = W.Workload("order", t, 64, "bf16", False, e, 1, k, mask_frac=mask, seed=seed)
    return W.make_topk(w)


def _case(t, k, e, r, a, row_bytes, s, seed, mask=0.05, flags=M.ALL_OUTPUTS, combined=False, row_order=True,
          **kw):
    print(f"\n[row-order] T={t} K={k} E={e} R={r} A={a} row={row_bytes} S={s} flags={flags} "
          f"combined={combined} order={row_order}", flush=True)
    topk = _topk(seed, t, k, e, mask)
    xb = H.random_rows(seed, t, row_bytes)
    sf = None if s == 0 else np.random.default_rng([seed, 7]).uniform(0.5, 2, (t, s)).astype(np.float32)
    ref = oracle.layout(topk, e, r, a, recv_capacity=kw.get("recv_capacity"),
                        rank_capacity=kw.get("rank_capacity"))
    run = H.run_gpu(topk, e, r, a, xb, sf, flags=flags, combined=combined, row_order=row_order, **kw)
    H.assert_layout_equal(run, ref)
    if ref.status == 0:
        H.assert_rows_full(run, ref, xb, sf)
    return run, ref


# Row widths around the ordered kernel's slicing: 4 KB (one slice of 256
# vectors), 4112 B (two slices of 129 and 128 vectors, 3 vectors per lane),
# 6160 B (two slices of 193 and 192), 7 KB and 8 KB (two slices of 224 and
# 256); alignment pads, scale factors, odd top-k, several tiles with a ragged
# tail, a one-tile batch. Rows beyond 8 KB keep no row order (its entry count
# is -1) and take the source-major scatter.
@pytest.mark.parametrize("t,k,e,r,a,row_bytes,s", [
    (300, 8, 64, 8, 1, 4096, 0),
    (513, 6, 48, 4, 16, 4112, 5),
    (1000, 8, 256, 8, 128, 7168, 56),
    (700, 3, 12, 3, 3, 8192, 0),
    (901, 5, 40, 5, 2, 6160, 1),
    (64, 8, 256, 8, 128, 7168, 56),
    (5, 2, 8, 2, 1, 4096, 70),
    (1500, 8, 256, 8, 1, 14336, 0),
])
@pytest.mark.parametrize("combined", [False, True], ids=["two_calls", "one_call"])
def test_ordered_scatter_shapes(t, k, e, r, a, row_bytes, s, combined):
    _case(t, k, e, r, a, row_bytes, s, seed=t + k, combined=combined)


@pytest.mark.parametrize("flags", [M.RANK_CONTIG, M.EXPERT_MAJOR, M.EXPERT_MAJOR | M.ZERO_PAD,
                                   M.RANK_CONTIG | M.EXPERT_MAJOR])
def test_ordered_scatter_output_selection(flags):
    # Rank rows alone are one destination per token: no row order is kept.
    _case(400, 8, 64, 8, 8, 4096, 3, seed=41, flags=flags)


def test_no_row_order_beyond_the_read_ahead():
    """Rows that the layout does not read ahead (above 160 MB) keep no row
    order: every destination would re-read its source row from HBM."""
    run, _ = _case(25000, 8, 256, 8, 1, 7168, 0, seed=45)
    assert int(run.layout.row_order[0].item()) == -1


def test_ordered_scatter_fully_masked_tokens_and_empty_batch():
    topk = _topk(42, 200, 8, 64, 0.0)
    topk[10:30] = -1
    xb = H.random_rows(42, 200, 4096)
    ref = oracle.layout(topk, 64, 8, 4)
    run = H.run_gpu(topk, 64, 8, 4, xb)
    H.assert_layout_equal(run, ref)
    H.assert_rows_full(run, ref, xb, None)
    _case(0, 8, 64, 8, 4, 4096, 0, seed=43)


def test_ordered_scatter_writes_nothing_on_overflow():
    topk = _topk(44, 600, 8, 64, 0.0)
    full = oracle.layout(topk, 64, 8, 4)
    run, ref = _case(600, 8, 64, 8, 4, 4096, 0, seed=44, mask=0.0, recv_capacity=full.num_recv_rows - 1)
    assert ref.status == oracle.RECV_OVERFLOW
    for name in ("rank_x", "recv_x"):
        assert np.all(getattr(run.rows, name).cpu().numpy() == H.ROW_FILL)


# The same shapes without a row order: the source-major scatter.
@pytest.mark.parametrize("t,k,e,r,a,row_bytes,s", [
    (513, 6, 48, 4, 16, 4112, 5),
    (1000, 8, 256, 8, 128, 7168, 56),
    (1500, 8, 256, 8, 1, 14336, 0),
])
def test_source_major_scatter_without_row_order(t, k, e, r, a, row_bytes, s):
    run, _ = _case(t, k, e, r, a, row_bytes, s, seed=t + 1, row_order=False)
    assert run.layout.row_order is None
