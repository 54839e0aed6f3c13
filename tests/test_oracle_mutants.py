"""Planted mistakes in a copy of the CPU oracle must fail the pins (CPU only).

Each mutant is the oracle's C source with one plausible mistake written in (a
dropped alignment, the wrong rounding, the wrong dedup owner, an off-by-one
cursor, reversed token order, interleaved ranks, unmarked pads, a wrong copy
source, a skipped zero fill). It is compiled into a temporary library and run
on a few inputs; the pin checks must reject every mutant. This shows the pins
are sharp enough to catch such mistakes in the real oracle.
"""

import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dispatch_oracle.c")

LAYOUT_MUTANTS = {
    "no_alignment": ("run += align_up(expert_count[e], A);", "run += expert_count[e];", 2),
    "floor_alignment": ("return ((c + a - 1) / a) * a;", "return (c / a) * a;", 1),
    "lowest_k_owns_rank_slot": (
        "            for (int32_t j = k + 1; j < K; ++j)\n"
        "                if (is_routed(row[j], E) && row[j] / experts_per_rank == r) owner = 0;\n"
        "            if (owner) {",
        "            for (int32_t j = 0; j < k; ++j)\n"
        "                if (is_routed(row[j], E) && row[j] / experts_per_rank == r) owner = 0;\n"
        "            if (owner) {", 1),
    "no_rank_dedup": ("if (owner) rank_count[r] += 1;", "rank_count[r] += 1;", 1),
    "cursor_off_by_one": ("expert_cursor[e] = expert_psum[e];", "expert_cursor[e] = expert_psum[e] + 1;", 1),
    "rank_cursor_off_by_one": ("rank_cursor[r] = rank_psum[r];", "rank_cursor[r] = rank_psum[r] + (r > 0);", 1),
    "reversed_token_order": (
        "    for (int64_t t = 0; t < T; ++t) {\n        const int64_t* row = topk_idx + t * K;\n"
        "        for (int32_t k = 0; k < K; ++k) {\n            const int64_t e = row[k];\n"
        "            if (e < 0) {",
        "    for (int64_t t = T - 1; t >= 0; --t) {\n        const int64_t* row = topk_idx + t * K;\n"
        "        for (int32_t k = 0; k < K; ++k) {\n            const int64_t e = row[k];\n"
        "            if (e < 0) {", 1),
    "interleaved_ranks": ("const int64_t r = e / experts_per_rank;", "const int64_t r = e % R;", 2),
    "pads_not_marked": ("recv_src_token_idx[s] = -1;", "recv_src_token_idx[s] = 0;", 1),
    "psum_lags_one_expert": ("        run += align_up(expert_count[e], A);\n        expert_psum[e + 1] = (int32_t)run;",
                             "        expert_psum[e + 1] = (int32_t)run;\n        run += align_up(expert_count[e], A);", 2),
}

SCATTER_MUTANTS = {
    "wrong_source_row": ("memcpy(recv_x + slot * row_bytes, x + t * row_bytes",
                         "memcpy(recv_x + slot * row_bytes, x + ((t + 1) % T) * row_bytes", 1),
    "rank_rows_skip_first_token": ("const int64_t row = rank_slot[t * K + k];",
                                   "const int64_t row = t == 0 ? -1 : rank_slot[t * K + k];", 1),
    "no_zero_pad": ("if (recv_x) memset(recv_x + s * row_bytes, 0, (size_t)row_bytes);", "(void)0;", 1),
    "sf_short_copy": ("memcpy(recv_sf + slot * S, x_sf + t * S, sf_bytes);",
                      "memcpy(recv_sf + slot * S, x_sf + t * S, sf_bytes - 4);", 1),
}


def _mutant_lib(tmp_path, name, old, new, count):
    src = open(SRC).read()
    assert src.count(old) == count, f"{name}: pattern found {src.count(old)} times"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(path), so)
    return oracle.load_library(so)


def _cases():
    rng = np.random.default_rng(5)
    out = []
    for t, k, e, r, a in [(37, 4, 16, 4, 4), (64, 6, 12, 3, 3), (20, 3, 8, 2, 1), (50, 8, 32, 8, 8)]:
        g = rng.gumbel(size=(t, e))
        topk = np.argsort(-g, axis=1, kind="stable")[:, :k].astype(np.int64)
        topk[rng.random((t, k)) < 0.15] = -1
        out.append((topk, e, r, a))
    w = W.get("tiny")
    out.append((W.make_topk(w), w.num_experts, w.num_ranks, w.alignment))
    return out


def _layout_rejected(lib):
    for topk, e, r, a in _cases():
        # Spare capacity keeps an off-by-one mutant's stray write inside the
        # arrays, where the canary check sees it.
        mr, mk = oracle.max_rows(topk.shape[0], topk.shape[1], e, r, a)
        try:
            lay = oracle.layout(topk, e, r, a, recv_capacity=mr + 64, rank_capacity=mk + 64, lib=lib)
            pins.check_layout(topk, e, r, a, lay, canary=oracle.CANARY)
            pins.check_against_brute_force(topk, e, r, a, lay)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(LAYOUT_MUTANTS))
def test_layout_mutant_is_caught(tmp_path, name):
    lib = _mutant_lib(tmp_path, name, *LAYOUT_MUTANTS[name])
    assert _layout_rejected(lib), f"pins did not catch mutant {name}"


@pytest.mark.parametrize("name", sorted(SCATTER_MUTANTS))
def test_scatter_mutant_is_caught(tmp_path, name):
    lib = _mutant_lib(tmp_path, name, *SCATTER_MUTANTS[name])
    rng = np.random.default_rng(9)
    caught = False
    for topk, e, r, a in _cases():
        t = topk.shape[0]
        x = rng.integers(0, 256, size=(t, 64), dtype=np.uint8)
        sf = rng.uniform(0.5, 2.0, size=(t, 3)).astype(np.float32)
        lay = oracle.layout(topk, e, r, a)
        rows = oracle.scatter(lay, x, sf, lib=lib)
        try:
            pins.check_rows(lay, x, sf, rows)
        except AssertionError:
            caught = True
            break
    assert caught, f"pins did not catch mutant {name}"


def test_unmutated_oracle_passes_same_cases(tmp_path):
    lib = _mutant_lib(tmp_path, "identity", "int status = 0;", "int status = 0;", 2)
    assert not _layout_rejected(lib)


EXPAND_MUTANTS = {
    "expand_reads_past_count": ("        for (int32_t i = 0; i < recv_count[s]; ++i) {\n            const int64_t r = (int64_t)s * M + i;",
                                "        for (int32_t i = 0; i < M; ++i) {\n            const int64_t r = (int64_t)s * M + i;", 1),
    "expand_sources_reversed": ("    for (int32_t s = 0; s < S; ++s) {\n        for (int32_t i = 0; i < recv_count[s]; ++i) {",
                                "    for (int32_t s = S - 1; s >= 0; --s) {\n        for (int32_t i = 0; i < recv_count[s]; ++i) {", 1),
    "expand_wrong_local_base": ("const int64_t first_expert = (int64_t)local_rank * L;",
                                "const int64_t first_expert = (int64_t)local_rank * L + (local_rank > 0);", 1),
}


@pytest.mark.parametrize("name", sorted(EXPAND_MUTANTS))
def test_expand_mutant_is_caught(tmp_path, name):
    from tests.test_oracle_pins import _expand_brute_force, _random_topk as rt

    lib = _mutant_lib(tmp_path, name, *EXPAND_MUTANTS[name])
    rng = np.random.default_rng(17)
    caught = False
    for trial in range(6):
        s_count, m, k, e, r = 3, 20, 4, 32, 4
        rank, a = trial % r, 1 + trial % 3
        recv_topk = np.concatenate([rt(rng, m, k, e, mask=0.1) for _ in range(s_count)])
        counts = rng.integers(5, m, size=s_count).astype(np.int32)
        got = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a, lib=lib)
        cnt, start, slot, src = _expand_brute_force(recv_topk, counts, s_count, m, e, r, rank, a)
        if (got.status != 0 or not np.array_equal(got.expert_count, cnt) or not np.array_equal(got.expert_psum, start)
                or not np.array_equal(got.expert_slot.astype(np.int64), slot)):
            caught = True
            break
    assert caught, f"pins did not catch mutant {name}"


COMBINE_MUTANTS = {
    "combine_ignores_weight": ("const double w = (double)weights[t * num_topk + k];", "const double w = 1.0;", 1),
    "combine_skips_first_k": ("        for (int32_t k = 0; k < num_topk; ++k) {\n            const int64_t slot = expert_slot[t * num_topk + k];",
                              "        for (int32_t k = 1; k < num_topk; ++k) {\n            const int64_t slot = expert_slot[t * num_topk + k];", 1),
    "combine_float_accumulate": ("o[h] += w * bf16_value(row[h]);", "o[h] = (float)(o[h] + (float)w * (float)bf16_value(row[h]));", 1),
}


@pytest.mark.parametrize("name", sorted(COMBINE_MUTANTS))
def test_combine_mutant_is_caught(tmp_path, name):
    from tests import test_oracle_pins as P

    lib = _mutant_lib(tmp_path, name, *COMBINE_MUTANTS[name])
    caught = False
    for seed in range(3):
        topk, lay, y, wts = P._combine_case(seed)
        got = oracle.combine(y, wts, lay.expert_slot, lib=lib)
        yv = P._bf16_bits_to_f64(y)
        slots = lay.expert_slot
        want = np.zeros((slots.shape[0], y.shape[1]))
        for kk in range(slots.shape[1]):
            valid = slots[:, kk] >= 0
            want[valid] += wts[valid, kk].astype(np.float64)[:, None] * yv[slots[valid, kk]]
        if not np.allclose(got, want, rtol=1e-13, atol=1e-300):
            caught = True
            break
    assert caught, f"pins did not catch mutant {name}"
