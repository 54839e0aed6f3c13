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


# ---------------------------------------------------------------- receiver-side expand


def _receive_from_one_source(topk, num_experts, num_ranks, rank, spare=7):
    """The rows rank `rank` receives from a single source, laid out like a
    fixed-stride receive buffer with `spare` unused rows after them."""
    lay = oracle.layout(topk, num_experts, num_ranks, 1)
    lo, hi = int(lay.rank_psum[rank]), int(lay.rank_psum[rank + 1])
    tokens = lay.rank_src_token_idx[lo:hi].astype(np.int64)
    m = (hi - lo) + spare
    recv_topk = np.full((m, topk.shape[1]), 12345, dtype=np.int64)  # junk in unused rows
    recv_topk[: hi - lo] = topk[tokens]
    return lay, tokens, recv_topk, np.array([hi - lo], dtype=np.int32), m


@pytest.mark.parametrize("seed", range(4))
def test_expand_single_source_equals_sender_expert_major_slice(seed):
    """With one source, the receiver's expert-major layout over its local
    experts equals the sender's expert-major layout restricted to that rank's
    experts (the page's expand builds the same buckets, sections 6.4 and 8.2)."""
    rng = np.random.default_rng([91, seed])
    e, r, k, t = 64, 8, 6, 300
    topk = _random_topk(rng, t, k, e, mask=0.1)
    a = int(rng.choice([1, 4, 16]))
    for rank in range(r):
        send, tokens, recv_topk, counts, m = _receive_from_one_source(topk, e, r, rank)
        sender = oracle.layout(topk, e, r, a)
        got = oracle.expand_layout(recv_topk, counts, 1, m, e, r, rank, a)
        assert got.status == 0
        L = e // r
        assert np.array_equal(got.expert_count, sender.expert_count[rank * L:(rank + 1) * L])
        base = int(sender.expert_psum[rank * L])
        assert np.array_equal(got.expert_psum, sender.expert_psum[rank * L:(rank + 1) * L + 1] - base)
        p = got.num_recv_rows
        src = got.recv_src_row_idx[:p]
        mapped = np.where(src >= 0, tokens[np.maximum(src, 0)], -1)
        assert np.array_equal(mapped, sender.recv_src_token_idx[base:base + p])
        # the pair slots agree too, through the received-row -> token map
        for i, tok in enumerate(tokens):
            for kk in range(k):
                ge = topk[tok, kk]
                if rank * L <= ge < (rank + 1) * L:
                    assert got.expert_slot[i, kk] == sender.expert_slot[tok, kk] - base
                else:
                    assert got.expert_slot[i, kk] == -1


def _expand_brute_force(recv_topk, counts, s_count, m, e, r, rank, a):
    L = e // r
    lo = rank * L
    pairs = [(s * m + i, kk, int(recv_topk[s * m + i, kk]) - lo)
             for s in range(s_count) for i in range(int(counts[s])) for kk in range(recv_topk.shape[1])
             if lo <= recv_topk[s * m + i, kk] < lo + L]
    cnt = [sum(1 for p in pairs if p[2] == x) for x in range(L)]
    span = []
    for c in cnt:
        q = 0
        while q < c:
            q += a
        span.append(q)
    start = [sum(span[:x]) for x in range(L + 1)]
    slot = np.full(recv_topk.shape, -1, dtype=np.int64)
    src = [-1] * start[-1]
    for x in range(L):
        q = start[x]
        for row, kk, ex in pairs:  # already in (source, row, k) order
            if ex == x:
                slot[row, kk] = q
                src[q] = row
                q += 1
    return np.array(cnt), np.array(start), slot, np.array(src, dtype=np.int64)


@pytest.mark.parametrize("seed", range(5))
def test_expand_multi_source_brute_force(seed):
    rng = np.random.default_rng([92, seed])
    s_count, m, k, e, r = int(rng.integers(1, 5)), int(rng.integers(0, 40)), 4, 32, 4
    rank, a = int(rng.integers(0, r)), int(rng.choice([1, 3, 8]))
    recv_topk = np.full((s_count * m, k), -1, dtype=np.int64)
    counts = rng.integers(0, m + 1, size=s_count).astype(np.int32)
    for s in range(s_count):
        blk = _random_topk(rng, m, k, e, mask=0.15)
        recv_topk[s * m:(s + 1) * m] = blk
    got = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a)
    assert got.status == 0
    cnt, start, slot, src = _expand_brute_force(recv_topk, counts, s_count, m, e, r, rank, a)
    assert np.array_equal(got.expert_count, cnt)
    assert np.array_equal(got.expert_psum, start)
    assert np.array_equal(got.expert_slot.astype(np.int64), slot)
    assert np.array_equal(got.recv_src_row_idx[:start[-1]].astype(np.int64), src)
    assert np.all(got.recv_src_row_idx[start[-1]:] == oracle.CANARY)


def test_expand_status_bits():
    recv_topk = np.array([[0, 1], [2, 3], [0, 2], [1, 3]], dtype=np.int64)
    counts = np.array([2, 2], dtype=np.int32)
    assert oracle.expand_layout(recv_topk, counts, 2, 2, 4, 2, 0, 1).status == 0
    assert oracle.expand_layout(recv_topk, np.array([3, 2], np.int32), 2, 2, 4, 2, 0, 1).status == oracle.BAD_COUNT
    assert oracle.expand_layout(recv_topk, np.array([-1, 2], np.int32), 2, 2, 4, 2, 0, 1).status == oracle.BAD_COUNT
    bad = recv_topk.copy()
    bad[1, 0] = 4
    assert oracle.expand_layout(bad, counts, 2, 2, 4, 2, 0, 1).status == oracle.BAD_EXPERT
    dup = recv_topk.copy()
    dup[0, 1] = 0  # local expert 0 twice in one row
    assert oracle.expand_layout(dup, counts, 2, 2, 4, 2, 0, 1).status == oracle.DUP_EXPERT
    dup_remote = recv_topk.copy()
    dup_remote[1] = [3, 3]  # another rank's expert twice: not this receiver's concern
    assert oracle.expand_layout(dup_remote, counts, 2, 2, 4, 2, 0, 1).status == 0
    # rank 0 owns experts 0, 1: rows 0 (0, 1), 2 (0), 3 (1) -> 4 pairs
    assert oracle.expand_layout(recv_topk, counts, 2, 2, 4, 2, 0, 1, recv_capacity=3).status == oracle.RECV_OVERFLOW
    # rows past a source's count are never read, whatever they hold
    junk = recv_topk.copy()
    junk[1] = [99, 99]
    assert oracle.expand_layout(junk, np.array([1, 2], np.int32), 2, 2, 4, 2, 0, 1).status == 0


# ---------------------------------------------------------------- combine


def _bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _combine_case(seed, t=64, k=6, e=32, h=40, mask=0.2):
    rng = np.random.default_rng([93, seed])
    topk = _random_topk(rng, t, k, e, mask=mask)
    lay = oracle.layout(topk, e, 4, 3)
    rows = lay.num_recv_rows
    y = rng.integers(0, 1 << 16, size=(rows, h), dtype=np.uint16)
    y[(y & 0x7F80) == 0x7F80] = 0x3F80  # no inf / nan patterns
    wts = rng.uniform(0.0, 1.0, size=(t, k)).astype(np.float32)
    return topk, lay, y, wts


@pytest.mark.parametrize("seed", range(4))
def test_combine_matches_numpy_gather_sum(seed):
    topk, lay, y, wts = _combine_case(seed)
    got = oracle.combine(y, wts, lay.expert_slot)
    yv = _bf16_bits_to_f64(y)
    slots = lay.expert_slot
    want = np.zeros((slots.shape[0], y.shape[1]))
    for kk in range(slots.shape[1]):
        valid = slots[:, kk] >= 0
        want[valid] += wts[valid, kk].astype(np.float64)[:, None] * yv[slots[valid, kk]]
    assert np.allclose(got, want, rtol=1e-13, atol=1e-300)


def test_combine_one_hot_weights_give_rows_exactly():
    topk, lay, y, wts = _combine_case(7)
    slots = lay.expert_slot
    one_hot = np.zeros_like(wts)
    first_valid = np.argmax(slots >= 0, axis=1)
    has = (slots >= 0).any(axis=1)
    one_hot[np.arange(len(wts))[has], first_valid[has]] = 1.0
    got = oracle.combine(y, one_hot, slots)
    yv = _bf16_bits_to_f64(y)
    for t in range(len(wts)):
        want = yv[slots[t, first_valid[t]]] if has[t] else np.zeros(y.shape[1])
        assert np.array_equal(got[t], want)


def test_combine_linearity_masking_and_order():
    topk, lay, y, wts = _combine_case(8)
    slots = lay.expert_slot
    base = oracle.combine(y, wts, slots)
    assert np.array_equal(oracle.combine(y, wts * 2, slots), base * 2)  # exact in binary
    assert not oracle.combine(y, wts, np.full_like(slots, -1)).any()
    perm = np.random.default_rng(1).permutation(slots.shape[1])
    assert np.allclose(oracle.combine(y, wts[:, perm], slots[:, perm]), base, rtol=1e-13, atol=1e-300)


def test_combine_of_scatter_is_weighted_identity():
    """Expert outputs equal to the dispatched rows (identity experts): combine
    brings every token back as x[t] times the sum of its routed weights."""
    w = W.Workload("id", 120, 64, "bf16", False, 32, 4, 4, mask_frac=0.1, alignment=8, seed=13)
    inp = W.make_inputs(w)
    lay = oracle.layout(inp.topk_idx, 32, 4, 8)
    rows = oracle.scatter(lay, inp.x_bytes())
    y = rows.recv_x.view(np.uint16)
    wts = W.make_topk_weights(w, inp.topk_idx)
    got = oracle.combine(y, wts, lay.expert_slot)
    x = _bf16_bits_to_f64(inp.x_bytes().view(np.uint16))
    scale = np.where(inp.topk_idx >= 0, wts.astype(np.float64), 0).sum(axis=1, keepdims=True)
    assert np.allclose(got, x * scale, rtol=1e-12, atol=1e-300)
    live = (inp.topk_idx >= 0).any(axis=1)
    assert np.allclose(scale[live], 1.0, atol=1e-6)
