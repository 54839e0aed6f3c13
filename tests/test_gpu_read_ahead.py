"""The scatter after a read-ahead layout, bit for bit against the CPU oracle:
dispatch_layout_read_ahead then dispatch_scatter with the
DISPATCH_ROWS_READ_AHEAD hint, and the combined call, which reads the rows
ahead and sets the hint itself when the rows fit the read-ahead. The hint
changes only the kernel (split_scatter_kernel instead of scatter_kernel) and
its launch (the reserved LDS that caps the workgroups per CU, from the
destinations per token); every output must equal the oracle's, with canary
bands past every total untouched."""

import numpy as np
import pytest

import moe_token_dispatch_amd as M
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _topk(seed, t, k, e, mask):
    w = W.Workload("read_ahead", t, 64, "bf16", False, e, 1, k, mask_frac=mask, seed=seed)
    return W.make_topk(w)


def _case(t, k, e, r, a, row_bytes, s, seed, mask=0.05, flags=M.ALL_OUTPUTS, combined=False, topk=None, **kw):
    print(f"\n[read-ahead] T={t} K={k} E={e} R={r} A={a} row={row_bytes} S={s} flags={flags} "
          f"combined={combined}", flush=True)
    topk = _topk(seed, t, k, e, mask) if topk is None else topk
    xb = H.random_rows(seed, t, row_bytes)
    sf = None if s == 0 else np.random.default_rng([seed, 7]).uniform(0.5, 2, (t, s)).astype(np.float32)
    ref = oracle.layout(topk, e, r, a, recv_capacity=kw.get("recv_capacity"),
                        rank_capacity=kw.get("rank_capacity"))
    run = H.run_gpu(topk, e, r, a, xb, sf, flags=flags, combined=combined, read_ahead=not combined, **kw)
    H.assert_layout_equal(run, ref)
    if ref.status == 0:
        H.assert_rows_full(run, ref, xb, sf)
    else:
        for name in ("rank_x", "recv_x"):
            buf = getattr(run.rows, name)
            if buf is not None:
                assert np.all(buf.cpu().numpy() == H.ROW_FILL), name
    return run, ref


# Destinations per token (K expert rows + min(K, R) rank rows) from 2 to 64,
# which set the wavefronts per workgroup and the workgroups per CU; row widths
# of one vector, a partial last 1 KB segment, whole segments, 7 KB fp8 rows
# with 56 scale factors and 14 KB rows; alignment pads; several layout tiles
# with a ragged tail.
@pytest.mark.parametrize("t,k,e,r,a,row_bytes,s", [
    (1000, 8, 256, 8, 128, 7168, 56),
    (513, 6, 48, 4, 16, 4112, 5),
    (700, 3, 12, 3, 3, 8192, 0),
    (901, 5, 40, 5, 2, 1040, 1),
    (600, 2, 8, 2, 1, 16, 0),
    (450, 16, 64, 8, 4, 2064, 3),
    (130, 32, 64, 32, 1, 1024, 0),
    (800, 1, 16, 4, 1, 4096, 2),
    (1500, 8, 256, 8, 1, 14336, 0),
])
@pytest.mark.parametrize("combined", [False, True], ids=["two_calls", "one_call"])
def test_read_ahead_scatter_shapes(t, k, e, r, a, row_bytes, s, combined):
    _case(t, k, e, r, a, row_bytes, s, seed=t + k, combined=combined)


@pytest.mark.parametrize("flags", [M.RANK_CONTIG, M.EXPERT_MAJOR, M.EXPERT_MAJOR | M.ZERO_PAD,
                                   M.RANK_CONTIG | M.EXPERT_MAJOR])
def test_read_ahead_output_selection(flags):
    _case(400, 8, 64, 8, 8, 4096, 3, seed=41, flags=flags)


def test_hint_beyond_the_read_ahead_is_ignored():
    """Rows that the layout does not read ahead (above 160 MB): the hint
    leaves the launch unbounded, and the rows are the oracle's."""
    _case(25000, 8, 256, 8, 1, 7168, 0, seed=45)


def test_fully_masked_tokens_and_empty_batch():
    topk = _topk(42, 200, 8, 64, 0.0)
    topk[10:30] = -1
    _case(200, 8, 64, 8, 4, 4096, 0, seed=42, topk=topk)
    _case(0, 8, 64, 8, 4, 4096, 0, seed=43)


def test_writes_nothing_on_overflow_or_bad_expert():
    topk = _topk(44, 600, 8, 64, 0.0)
    full = oracle.layout(topk, 64, 8, 4)
    _, ref = _case(600, 8, 64, 8, 4, 4096, 0, seed=44, topk=topk, recv_capacity=full.num_recv_rows - 1)
    assert ref.status == oracle.RECV_OVERFLOW
    bad = topk.copy()
    bad[77, 2] = 64
    _, ref = _case(600, 8, 64, 8, 4, 4096, 0, seed=46, topk=bad)
    assert ref.status == oracle.BAD_EXPERT
