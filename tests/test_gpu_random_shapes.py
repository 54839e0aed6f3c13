"""Seeded random problems, each compared bit for bit with the CPU oracle.

The hand-picked cases elsewhere pin the edges; these draw the parameters
together (tokens, top-k, experts, ranks, alignment, row width, scale factors,
routing width, masking, output selection), so that combinations no list
names still get checked. The draws are fixed by their seed.
"""

import numpy as np
import pytest

import moe_token_dispatch_amd as M
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

CASES = 24


def _draw(seed):
    rng = np.random.default_rng([seed, 2024])
    k = int(rng.choice([1, 2, 3, 4, 6, 8, 9, 16, 32]))
    r = int(rng.choice([1, 2, 4, 8, 16, 64, 256]))
    epr = int(rng.choice([1, 2, 4, 8, 32]))
    e = min(r * epr, 4096)
    e -= e % r
    e = max(e, r)
    k = min(k, e)
    t = int(rng.choice([0, 1, 7, 100, 257, 999, 3000, 9000, 20000]))
    a = int(rng.choice([1, 1, 2, 5, 16, 128]))
    row_bytes = int(rng.choice([16, 48, 256, 1040, 4096]))
    s = int(rng.choice([0, 0, 1, 3, 56]))
    topk_bytes = int(rng.choice([4, 8]))
    mask = float(rng.choice([0.0, 0.05, 0.5]))
    flags = int(rng.choice([M.ALL_OUTPUTS, M.ALL_OUTPUTS, M.EXPERT_MAJOR | M.ZERO_PAD, M.RANK_CONTIG,
                            M.EXPERT_MAJOR]))
    return t, k, e, r, a, row_bytes, s, topk_bytes, mask, flags


@pytest.mark.parametrize("seed", range(CASES))
def test_random_problem_matches_oracle(seed):
    t, k, e, r, a, row_bytes, s, topk_bytes, mask, flags = _draw(seed)
    print(f"\n[gpu-random] seed={seed} T={t} K={k} E={e} R={r} A={a} row={row_bytes} S={s} "
          f"idx={topk_bytes} mask={mask} flags={flags}", flush=True)
    w = W.Workload(f"rand{seed}", t, 64, "bf16", False, e, r, k, mask_frac=mask, seed=1000 + seed)
    topk = W.make_topk(w)
    xb = H.random_rows(seed, t, row_bytes)
    sf = None if s == 0 else np.random.default_rng([seed, 7]).uniform(0.5, 2, (t, s)).astype(np.float32)
    ref = oracle.layout(topk, e, r, a)
    assert ref.status == 0
    run = H.run_gpu(topk, e, r, a, xb, sf, topk_bytes=topk_bytes, flags=flags)
    H.assert_layout_equal(run, ref)
    H.assert_rows_full(run, ref, xb, sf)


ONE_CALL_CASES = 16


@pytest.mark.parametrize("seed", range(ONE_CALL_CASES))
def test_random_problem_through_the_one_call(seed):
    """The same draws, with the batch cut to the one kernel's limit (3072
    (token, k) pairs, 2048 when pad rows are zeroed) and run through
    dispatch_layout_and_scatter: one kernel where it fits, the layout and
    scatter kernels otherwise (many keys, few wavefronts)."""
    t, k, e, r, a, row_bytes, s, topk_bytes, mask, flags = _draw(500 + seed)
    pads = a > 1 and flags & M.EXPERT_MAJOR and flags & M.ZERO_PAD
    t = min(t, (2048 if pads else 3072) // k)
    print(f"\n[gpu-random] one call seed={seed} T={t} K={k} E={e} R={r} A={a} row={row_bytes} S={s} "
          f"idx={topk_bytes} mask={mask} flags={flags}", flush=True)
    w = W.Workload(f"rand1c{seed}", t, 64, "bf16", False, e, r, k, mask_frac=mask, seed=2000 + seed)
    topk = W.make_topk(w)
    xb = H.random_rows(seed, t, row_bytes)
    sf = None if s == 0 else np.random.default_rng([seed, 8]).uniform(0.5, 2, (t, s)).astype(np.float32)
    ref = oracle.layout(topk, e, r, a)
    assert ref.status == 0
    assert M.dispatch_kernel_count(M.make_problem(t, k, e, r, a, topk_bytes, row_bytes, s, flags=flags))[1] == 1
    run = H.run_gpu(topk, e, r, a, xb, sf, topk_bytes=topk_bytes, flags=flags, combined=True)
    H.assert_layout_equal(run, ref)
    H.assert_rows_full(run, ref, xb, sf)


SMALL_ALIGNED_CASES = 12


def _draw_small_aligned(seed):
    """Small batches over many experts with alignment: most fall where the
    scatter maps its pad wavefronts to row blocks, the rest just past it."""
    rng = np.random.default_rng([seed, 4242])
    r = int(rng.choice([1, 4, 8, 64]))
    e = int(rng.choice([64, 256, 1024, 4096]))
    e -= e % r
    k = int(rng.choice([1, 2, 4, 8]))
    t = int(rng.choice([1, 2, 5, 17, 40, 130]))
    a = int(rng.choice([2, 3, 16, 128]))
    row_bytes = int(rng.choice([16, 272, 1040, 7168]))
    s = int(rng.choice([0, 3, 56]))
    topk_bytes = int(rng.choice([4, 8]))
    mask = float(rng.choice([0.0, 0.2]))
    flags = int(rng.choice([M.ALL_OUTPUTS, M.EXPERT_MAJOR | M.ZERO_PAD]))
    return t, k, e, r, a, row_bytes, s, topk_bytes, mask, flags


@pytest.mark.parametrize("seed", range(SMALL_ALIGNED_CASES))
def test_random_small_aligned_batch(seed):
    t, k, e, r, a, row_bytes, s, topk_bytes, mask, flags = _draw_small_aligned(seed)
    print(f"\n[gpu-random] small aligned seed={seed} T={t} K={k} E={e} R={r} A={a} row={row_bytes} S={s} "
          f"idx={topk_bytes} mask={mask} flags={flags}", flush=True)
    w = W.Workload(f"randsa{seed}", t, 64, "bf16", False, e, r, k, mask_frac=mask, seed=3000 + seed)
    topk = W.make_topk(w)
    xb = H.random_rows(seed, t, row_bytes)
    sf = None if s == 0 else np.random.default_rng([seed, 9]).uniform(0.5, 2, (t, s)).astype(np.float32)
    ref = oracle.layout(topk, e, r, a)
    assert ref.status == 0
    run = H.run_gpu(topk, e, r, a, xb, sf, topk_bytes=topk_bytes, flags=flags)
    H.assert_layout_equal(run, ref)
    H.assert_rows_full(run, ref, xb, sf)
