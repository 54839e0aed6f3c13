"""Pins of the CPU oracle to facts other than itself (CPU only).

The oracle follows the "DeepEP Counting Sort / Bucketization" page. These
tests check it against the page's worked alignment example, closed forms,
numpy library routines (bincount, stable argsort, lexsort, index gathers),
brute-force enumeration on tiny inputs, exhaustive enumeration of every
2-token routing table of a small problem, and a closed-form expectation.
"""

import itertools
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    vals = {}
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0].isalpha() or "_" in parts[0]:
                vals[parts[0]] = int(parts[1])
            else:
                rows.append([int(p) for p in parts])
    return vals, rows


def _random_topk(rng, t, k, e, mask=0.0):
    g = rng.gumbel(size=(t, e))
    topk = np.argsort(-g, axis=1, kind="stable")[:, :k].astype(np.int64)
    if mask:
        topk[rng.random((t, k)) < mask] = -1
    return topk


def test_align_worked_example():
    """Section 7.3: 50 tokens under alignment 64 -> 64 slots, the last 14 zero pads."""
    v, _ = _read_fixture("align_worked_example.txt")
    n, a = v["expert_tokens"], v["alignment"]
    # Expert 2 of 4 receives n tokens (the page's figure uses expert 2); the
    # other experts receive a few so the bucket does not start at 0.
    e, r = 4, 2
    topk = np.full((n + 3, 1), 2, dtype=np.int64)
    topk[n:, 0] = [0, 1, 3]
    lay = oracle.layout(topk, e, r, a)
    assert lay.status == 0
    start, end = int(lay.expert_psum[2]), int(lay.expert_psum[3])
    assert end - start == v["aligned_slots"]
    bucket = lay.recv_src_token_idx[start:end]
    assert np.array_equal(bucket[:n], np.arange(n))
    assert int((bucket == -1).sum()) == v["pad_rows"]
    assert np.all(bucket[n:] == -1)
    x = np.random.default_rng(0).integers(1, 255, size=(n + 3, 32), dtype=np.uint8)
    rows = oracle.scatter(lay, x)
    assert not rows.recv_x[start + n:end].any()
    pins.check_rows(lay, x, None, rows)


def test_align_closed_form_table():
    """Section 7.2: align(a, b) = ceil(a / b) * b, as spans of single-expert problems."""
    _, rows = _read_fixture("align_closed_form.txt")
    for count, a, aligned in rows:
        topk = np.zeros((max(count, 1), 1), dtype=np.int64)
        if count == 0:
            topk[:] = 1  # every token goes to the other expert
        lay = oracle.layout(topk, 2, 1, a)
        assert int(lay.expert_psum[1] - lay.expert_psum[0]) == aligned, (count, a)


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_workload_layout_pins(name):
    w = W.get(name)
    topk = W.make_topk(w)
    lay = oracle.layout(topk, w.num_experts, w.num_ranks, w.alignment)
    pins.check_layout(topk, w.num_experts, w.num_ranks, w.alignment, lay, canary=oracle.CANARY)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_random(seed):
    rng = np.random.default_rng([77, seed])
    e = int(rng.choice([4, 8, 12, 16]))
    r = int(rng.choice([d for d in (1, 2, 4) if e % d == 0]))
    k = int(rng.integers(1, min(e, 6) + 1))
    t = int(rng.integers(0, 40))
    a = int(rng.choice([1, 2, 3, 4, 8]))
    topk = _random_topk(rng, t, k, e, mask=0.2)
    lay = oracle.layout(topk, e, r, a)
    pins.check_layout(topk, e, r, a, lay, canary=oracle.CANARY)
    pins.check_against_brute_force(topk, e, r, a, lay)


def _legal_rows(e, k):
    """Every legal routing row: k entries, each an expert or -1, experts distinct."""
    out = []
    for row in itertools.product(range(-1, e), repeat=k):
        used = [v for v in row if v >= 0]
        if len(used) == len(set(used)):
            out.append(row)
    return out


def test_exhaustive_two_tokens():
    """T=2, K=2, E=4, R=2: all 21 x 21 legal tables, alignments 1, 2 and 3."""
    rows = _legal_rows(4, 2)
    assert len(rows) == 21  # 12 ordered distinct pairs + 8 half-masked + 1 fully masked
    for a in (1, 2, 3):
        for r0, r1 in itertools.product(rows, rows):
            topk = np.array([r0, r1], dtype=np.int64)
            lay = oracle.layout(topk, 4, 2, a)
            pins.check_against_brute_force(topk, 4, 2, a, lay)
            pins.check_slots(topk, 4, 2, lay, canary=oracle.CANARY)


@pytest.mark.slow
def test_exhaustive_three_tokens():
    """T=3, K=2, E=4, R=2: all 9261 legal tables at alignment 2."""
    rows = _legal_rows(4, 2)
    for tbl in itertools.product(rows, rows, rows):
        topk = np.array(tbl, dtype=np.int64)
        lay = oracle.layout(topk, 4, 2, 2)
        pins.check_against_brute_force(topk, 4, 2, 2, lay)


def test_distinct_ranks_expectation():
    """Uniform top-8 of 256 experts in 8 ranks: E[distinct ranks per token] in closed form."""
    w = W.Workload("u", 4096, 128, "bf16", False, 256, 8, 8, seed=11)
    topk = W.make_topk(w)
    lay = oracle.layout(topk, 256, 8, 1)
    epr = 32
    # P(rank r untouched) = C(E - epr, K) / C(E, K); mean = R * (1 - that).
    expect = 8 * (1 - math.comb(256 - epr, 8) / math.comb(256, 8))
    assert abs(expect - 5.2947) < 1e-3
    mean = lay.rank_count.sum() / 4096
    assert abs(mean - expect) < 0.06, (mean, expect)


def test_fully_masked_and_empty():
    lay = oracle.layout(np.zeros((0, 4), np.int64), 8, 2, 4)
    assert lay.status == 0 and lay.expert_psum[-1] == 0 and lay.rank_psum[-1] == 0
    topk = np.full((5, 3), -1, np.int64)
    lay = oracle.layout(topk, 8, 2, 4)
    assert lay.status == 0 and not lay.expert_count.any() and not lay.rank_count.any()
    assert np.all(lay.expert_slot == -1) and np.all(lay.rank_slot == -1)


def test_any_negative_is_masked():
    topk = np.array([[-1, 3], [-5, 2], [0, -100]], dtype=np.int64)
    lay = oracle.layout(topk, 4, 2, 1)
    pins.check_layout(np.where(topk < 0, -1, topk), 4, 2, 1, lay)


def test_status_bits():
    ok = np.array([[0, 1], [2, 3]], dtype=np.int64)
    assert oracle.layout(ok, 4, 2, 1).status == 0
    bad = np.array([[0, 4], [2, 3]], dtype=np.int64)
    assert oracle.layout(bad, 4, 2, 1).status == oracle.BAD_EXPERT
    dup = np.array([[1, 1], [2, 3]], dtype=np.int64)
    assert oracle.layout(dup, 4, 2, 1).status == oracle.DUP_EXPERT
    # 4 routed pairs need 4 expert-major rows; token 0 only touches rank 0 and
    # token 1 only rank 1, so 2 rank rows.
    assert oracle.layout(ok, 4, 2, 1, recv_capacity=3).status == oracle.RECV_OVERFLOW
    assert oracle.layout(ok, 4, 2, 1, rank_capacity=1).status == oracle.RANK_OVERFLOW
    assert oracle.layout(ok, 4, 2, 1, recv_capacity=4, rank_capacity=2).status == 0
    with pytest.raises(ValueError):
        oracle.layout(ok, 4, 3, 1)  # E % R != 0
    with pytest.raises(ValueError):
        oracle.layout(np.zeros((1, 33), np.int64), 64, 1, 1)  # K > 32


@pytest.mark.parametrize("name", ["tiny", "dsv3_fp8_a128"])
def test_rows_match_library_gather(name):
    w = W.get(name)
    inp = W.make_inputs(w)
    lay = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment)
    rows = oracle.scatter(lay, inp.x_bytes(), inp.x_sf)
    pins.check_rows(lay, inp.x_bytes(), inp.x_sf, rows)


def test_rows_fp8_nan_payload_survives():
    """Copies are bitwise: fp8 NaN encodings (0x7f, 0xff) come through unchanged."""
    rng = np.random.default_rng(3)
    topk = _random_topk(rng, 16, 2, 8)
    x = rng.integers(0, 256, size=(16, 48), dtype=np.uint8)
    x[:, 0] = 0x7F
    x[:, 1] = 0xFF
    lay = oracle.layout(topk, 8, 4, 4)
    rows = oracle.scatter(lay, x)
    pins.check_rows(lay, x, None, rows)
