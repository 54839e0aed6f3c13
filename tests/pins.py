"""Checks that pin a dispatch layout to facts other than the oracle itself.

Each check uses a different formulation from the oracle's cursor walk: numpy
library routines (bincount, stable argsort, lexsort, unique, index gathers),
brute-force enumeration and the properties the "DeepEP Counting Sort /
Bucketization" page states. Every check raises AssertionError on a mismatch,
so the same functions serve the oracle's tests and the mutation tests that
plant mistakes in a copy of the oracle.
"""

from __future__ import annotations

import numpy as np
import torch


def valid_pairs(topk: np.ndarray):
    """(token, expert, flat index) of every routed pair, in (t, k) order."""
    t_count, k = topk.shape
    flat_e = topk.reshape(-1)
    keep = flat_e >= 0
    t_of = np.repeat(np.arange(t_count, dtype=np.int64), k)
    return t_of[keep], flat_e[keep].astype(np.int64), np.nonzero(keep)[0]


def check_counts(topk, num_experts, num_ranks, lay):
    t, e, _ = valid_pairs(topk)
    # Every routed pair counts once for its expert (no dedup, section 4.2).
    assert np.array_equal(lay.expert_count, np.bincount(e, minlength=num_experts)), "expert_count"
    assert int(lay.expert_count.sum()) == len(e), "sum of expert counts != routed pairs"
    # A rank counts each token once (dedup, section 4.2): distinct (t, r) pairs.
    epr = num_experts // num_ranks
    tr = np.unique(t * num_ranks + e // epr)
    assert np.array_equal(lay.rank_count, np.bincount(tr % num_ranks, minlength=num_ranks)), "rank_count"
    # A rank sees at least its busiest expert's tokens and at most the sum.
    ec = lay.expert_count.reshape(num_ranks, epr)
    assert np.all(ec.max(axis=1) <= lay.rank_count), "rank_count below an expert count"
    assert np.all(lay.rank_count <= ec.sum(axis=1)), "rank_count above the expert sum"


def _round_up_by_search(c: np.ndarray, a: int) -> np.ndarray:
    """Smallest multiple of a that is >= c, found by searching the list of multiples."""
    c = np.asarray(c, dtype=np.int64)
    top = int(c.max()) if c.size else 0
    multiples = np.arange(0, top + 2 * a, a, dtype=np.int64)
    return multiples[np.searchsorted(multiples, c, side="left")]


def check_psums(lay, alignment):
    a = max(int(alignment), 1)
    p = lay.expert_psum.astype(np.int64)
    c = lay.expert_count.astype(np.int64)
    assert p[0] == 0, "expert_psum[0] != 0"
    d = np.diff(p)
    # The span of each expert is a multiple of A that holds all its rows with
    # fewer than A pads: that is exactly align(count, A) (section 7.2).
    assert np.all(d % a == 0), "expert span not a multiple of the alignment"
    assert np.all(d >= c), "expert span shorter than its count"
    assert np.all(d < c + a), "expert span has A or more pads"
    assert np.array_equal(d, _round_up_by_search(c, a)), "expert span != stepped round-up"
    assert np.all(p % a == 0), "expert start not aligned"
    # Handle identities (section 10.2-10.3): with incl[e] = start[e] + count[e],
    # rounding incl[e] up gives the next expert's start, and incl[e] minus the
    # rounded-up incl[e-1] gives the real count.
    incl = p[:-1] + c
    assert np.array_equal(_round_up_by_search(incl, a), p[1:]), "align(incl[e]) != start[e+1]"
    if len(c) > 1:
        assert np.array_equal(incl[1:] - _round_up_by_search(incl[:-1], a), c[1:]), "incl identity"
    # Rank psum: exclusive, its last element is the total of rank rows (section 5.5).
    rp = lay.rank_psum.astype(np.int64)
    assert rp[0] == 0 and np.array_equal(np.diff(rp), lay.rank_count), "rank_psum"
    assert rp[-1] == lay.rank_count.sum(), "rank_psum total"


def check_slots(topk, num_experts, num_ranks, lay, canary=None):
    t, e, flat = valid_pairs(topk)
    p_total = int(lay.expert_psum[-1])
    n_rank = int(lay.rank_psum[-1])
    es = lay.expert_slot.reshape(-1).astype(np.int64)
    rs = lay.rank_slot.reshape(-1).astype(np.int64)
    masked = topk.reshape(-1) < 0
    assert np.all(es[masked] == -1) and np.all(rs[masked] == -1), "masked pair got a slot"

    # Expert-major order = a stable sort of the routed pairs by expert: inside
    # each bucket, ascending token index (then k, which cannot tie for one expert).
    order = np.argsort(e, kind="stable")
    e_sorted = e[order]
    within = np.arange(len(e)) - np.searchsorted(e_sorted, e_sorted, side="left")
    expected = np.empty(len(e), dtype=np.int64)
    expected[order] = lay.expert_psum.astype(np.int64)[e_sorted] + within
    assert np.array_equal(es[flat], expected), "expert_slot != stable-sort position"

    recv = lay.recv_src_token_idx[:p_total].astype(np.int64)
    assert np.all(recv[es[flat]] == t), "recv_src_token_idx does not invert expert_slot"
    assert np.array_equal(recv[recv >= 0], t[order]), "recv_src_token_idx != stable-sorted tokens"
    assert int((recv == -1).sum()) == p_total - len(e), "pad entries are not exactly the -1 entries"
    assert np.all((recv == -1) | (recv >= 0)), "recv_src_token_idx holds junk"

    # Rank-contiguous order: distinct (t, r) pairs sorted by rank, then token;
    # the slot sits at the highest k of that rank in the token (section 4.2's
    # master lane), the other k of the rank hold -1.
    epr = num_experts // num_ranks
    key = t * num_ranks + e // epr
    uniq, last_rev = np.unique(key[::-1], return_index=True)
    owner_flat = flat[len(key) - 1 - last_rev]
    holders = np.nonzero(rs >= 0)[0]
    assert np.array_equal(np.sort(holders), np.sort(owner_flat)), "rank slot not at the highest k"
    ut, ur = uniq // num_ranks, uniq % num_ranks
    o = np.lexsort((ut, ur))
    pos = np.empty(len(uniq), dtype=np.int64)
    pos[o] = np.arange(len(uniq))
    assert np.array_equal(rs[owner_flat], pos), "rank_slot != (rank, token) sort position"
    assert n_rank == len(uniq), "rank row total"
    assert np.array_equal(lay.rank_src_token_idx[:n_rank].astype(np.int64), ut[o]), "rank_src_token_idx"

    if canary is not None:
        assert np.all(lay.recv_src_token_idx[p_total:] == canary), "recv_src written past the total"
        assert np.all(lay.rank_src_token_idx[n_rank:] == canary), "rank_src written past the total"


def check_layout(topk, num_experts, num_ranks, alignment, lay, canary=None):
    assert lay.status == 0, f"unexpected status {lay.status}"
    check_counts(topk, num_experts, num_ranks, lay)
    check_psums(lay, alignment)
    check_slots(topk, num_experts, num_ranks, lay, canary)


def brute_force_layout(topk, num_experts, num_ranks, alignment):
    """O(E * T * K) enumeration, one expert (then one rank) at a time."""
    t_count, k_count = topk.shape
    epr = num_experts // num_ranks
    rows = topk.tolist()
    cnt = [sum(1 for t in range(t_count) for k in range(k_count) if rows[t][k] == e)
           for e in range(num_experts)]
    span = []
    for c in cnt:
        m = 0
        while m < c:
            m += max(alignment, 1)
        span.append(m)
    start = [sum(span[:e]) for e in range(num_experts + 1)]
    expert_slot = [[-1] * k_count for _ in range(t_count)]
    recv = [-1] * start[-1]
    for e in range(num_experts):
        s = start[e]
        for t in range(t_count):
            for k in range(k_count):
                if rows[t][k] == e:
                    expert_slot[t][k] = s
                    recv[s] = t
                    s += 1
    in_rank = [[[k for k in range(k_count) if rows[t][k] >= 0 and rows[t][k] // epr == r]
                for r in range(num_ranks)] for t in range(t_count)]
    rcnt = [sum(1 for t in range(t_count) if in_rank[t][r]) for r in range(num_ranks)]
    rstart = [sum(rcnt[:r]) for r in range(num_ranks + 1)]
    rank_slot = [[-1] * k_count for _ in range(t_count)]
    rank_src = [-1] * rstart[-1]
    for r in range(num_ranks):
        s = rstart[r]
        for t in range(t_count):
            if in_rank[t][r]:
                rank_slot[t][max(in_rank[t][r])] = s
                rank_src[s] = t
                s += 1
    return dict(expert_count=np.array(cnt), rank_count=np.array(rcnt),
                expert_psum=np.array(start), rank_psum=np.array(rstart),
                expert_slot=np.array(expert_slot).reshape(t_count, k_count),
                rank_slot=np.array(rank_slot).reshape(t_count, k_count),
                recv_src_token_idx=np.array(recv, dtype=np.int64),
                rank_src_token_idx=np.array(rank_src, dtype=np.int64))


def check_against_brute_force(topk, num_experts, num_ranks, alignment, lay):
    bf = brute_force_layout(topk, num_experts, num_ranks, alignment)
    for name in ("expert_count", "rank_count", "expert_psum", "rank_psum", "expert_slot", "rank_slot"):
        assert np.array_equal(getattr(lay, name).astype(np.int64), bf[name].astype(np.int64)), name
    p_total, n_rank = int(bf["expert_psum"][-1]), int(bf["rank_psum"][-1])
    assert np.array_equal(lay.recv_src_token_idx[:p_total].astype(np.int64), bf["recv_src_token_idx"]), "recv_src"
    assert np.array_equal(lay.rank_src_token_idx[:n_rank].astype(np.int64), bf["rank_src_token_idx"]), "rank_src"


def check_rows(lay, x_bytes, x_sf, rows):
    """Row bytes equal a library gather of x by the inverse maps; pads are zero."""
    p_total = int(lay.expert_psum[-1])
    n_rank = int(lay.rank_psum[-1])
    xb = torch.from_numpy(np.ascontiguousarray(x_bytes))
    recv = lay.recv_src_token_idx[:p_total].astype(np.int64)
    real = recv >= 0
    if rows.recv_x is not None:
        got = torch.from_numpy(np.ascontiguousarray(rows.recv_x))
        assert got.shape[0] == p_total
        want = torch.index_select(xb, 0, torch.from_numpy(recv[real]))
        assert torch.equal(got[torch.from_numpy(real)], want), "recv_x real rows"
        assert not bool(got[torch.from_numpy(~real)].any()), "recv_x pad rows not zero"
    if rows.rank_x is not None:
        got = torch.from_numpy(np.ascontiguousarray(rows.rank_x))
        src = torch.from_numpy(lay.rank_src_token_idx[:n_rank].astype(np.int64))
        assert torch.equal(got, torch.index_select(xb, 0, src)), "rank_x rows"
    if x_sf is not None:
        sfb = torch.from_numpy(np.ascontiguousarray(x_sf).view(np.int32))
        if rows.recv_sf is not None:
            got = torch.from_numpy(np.ascontiguousarray(rows.recv_sf).view(np.int32))
            want = torch.index_select(sfb, 0, torch.from_numpy(recv[real]))
            assert torch.equal(got[torch.from_numpy(real)], want), "recv_sf real rows"
            assert not bool(got[torch.from_numpy(~real)].any()), "recv_sf pad rows not zero"
        if rows.rank_sf is not None:
            got = torch.from_numpy(np.ascontiguousarray(rows.rank_sf).view(np.int32))
            src = torch.from_numpy(lay.rank_src_token_idx[:n_rank].astype(np.int64))
            assert torch.equal(got, torch.index_select(sfb, 0, src)), "rank_sf rows"
