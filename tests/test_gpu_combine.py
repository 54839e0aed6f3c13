"""GPU combine (weighted reverse gather over the expert-major slots) against
the CPU oracle, through the C ABI.

The oracle sums in double precision. The kernel widens bf16 to fp32, adds one
fused multiply-add per routed k (ascending k, from 0) and rounds the fp32 sum
to bf16 once. With A = sum_k |w_k| |y_k| and u = 2^-24, the K-term fp32 chain
is within K u A of the exact sum S (each FMA rounds once, to at most u times
its partial sum, which is at most A), and the final rounding adds at most half
a bf16 ulp, 2^-8 |S_fp32|. The test bound is therefore

    |gpu - S| <= 2^-8 (max(|gpu|, |S|) + (K+1) u A) + (K+1) u A + 2^-133

(the last term covers bf16's subnormal spacing). On top of that bound almost
every output must equal S rounded to bf16 exactly: the two differ only where
the fp32 error crosses a bf16 rounding boundary.
"""

import numpy as np
import pytest
import torch

import moe_token_dispatch_amd as M
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

U = H.U
_bf16_bits_to_f64 = H.bf16_bits_to_f64
_f64_to_bf16_rne = H.f64_to_bf16_rne
_check = H.assert_combine_close


def _banner(msg):
    print(f"\n[gpu-combine] {msg}", flush=True)


def _combine_inputs(t, k, e, hidden, mask, seed, alignment=1):
    w = W.Workload(f"comb{seed}", t, hidden, "bf16", False, e, max(1, e // 8), k, mask_frac=mask,
                   alignment=alignment, seed=seed)
    topk = W.make_topk(w)
    ref = oracle.layout(topk, e, w.num_ranks, alignment)
    assert ref.status == 0
    rows = max(ref.num_recv_rows, 1)
    y = W.make_expert_out(w, rows)
    wts = W.make_topk_weights(w, topk)
    return w, topk, ref, y, wts


def _run_combine(slots: np.ndarray, wts: np.ndarray, y: torch.Tensor) -> np.ndarray:
    t, hidden = slots.shape[0], y.shape[1]
    out = torch.full((t, hidden), -123.0, dtype=torch.bfloat16, device=H.DEVICE)
    M.dispatch_combine(torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).to(H.DEVICE),
                       torch.from_numpy(np.ascontiguousarray(wts, dtype=np.float32)).to(H.DEVICE),
                       y.to(H.DEVICE), out)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("t,k,e,hidden,mask", [
    (512, 8, 256, 7168, 0.05),    # 14 segments of 64 vectors
    (300, 8, 64, 4096, 0.0),      # 8 whole segments, no masking
    (257, 6, 32, 2056, 0.1),      # ragged: 4 segments and a 1-vector tail
    (129, 4, 16, 128, 0.3),       # 16 vectors: most lanes idle
    (65, 1, 8, 8, 0.2),           # one vector per row, top-1
    (96, 32, 64, 1024, 0.25),     # the largest top-k: 4 batches of 8 loads
    (100, 11, 64, 512, 0.0),      # a second batch of 3
])
def test_combine_matches_oracle(t, k, e, hidden, mask):
    _banner(f"combine T={t} K={k} E={e} H={hidden} mask={mask}")
    w, topk, ref, y, wts = _combine_inputs(t, k, e, hidden, mask, seed=hidden + k)
    y_bits = y.view(torch.int16).numpy().view(np.uint16)
    got = _run_combine(ref.expert_slot, wts, y)
    _check(got, y_bits, wts, ref.expert_slot)


def test_combine_one_hot_weights_copy_rows_exactly():
    _banner("one-hot weights")
    w, topk, ref, y, wts = _combine_inputs(200, 8, 64, 1032, 0.1, seed=11)
    slots = ref.expert_slot
    pick = np.argmax(slots >= 0, axis=1)
    one_hot = np.zeros_like(wts)
    has = (slots >= 0).any(axis=1)
    one_hot[np.arange(len(slots))[has], pick[has]] = 1.0
    got = _run_combine(slots, one_hot, y)
    y_bits = y.view(torch.int16).numpy().view(np.uint16)
    want = np.where(has[:, None], y_bits[np.maximum(slots[np.arange(len(slots)), pick], 0)], 0)
    assert np.array_equal(got, want)


def test_combine_masked_and_empty_tokens():
    _banner("fully masked tokens and T=0")
    w, topk, ref, y, wts = _combine_inputs(64, 4, 16, 256, 0.0, seed=12)
    slots = ref.expert_slot.copy()
    slots[::3] = -1                      # a third of the tokens route nowhere
    slots[1::3, :2] = -1
    got = _run_combine(slots, wts, y)
    _check(got, y.view(torch.int16).numpy().view(np.uint16), wts, slots)
    empty = _run_combine(np.zeros((0, 4), np.int32), np.zeros((0, 4), np.float32), y)
    assert empty.shape == (0, 256)


def test_combine_inverts_weighted_scatter_end_to_end():
    """GPU layout -> GPU scatter of x -> GPU combine gives bf16(x * sum_k w) for
    every token: the combine reads back exactly the rows the scatter wrote."""
    _banner("scatter then combine, aligned buckets")
    w = W.Workload("roundtrip", 777, 2048, "bf16", False, 64, 8, 8, mask_frac=0.1, alignment=16, seed=21)
    inp = W.make_inputs(w)
    run = H.run_gpu(inp.topk_idx, w.num_experts, w.num_ranks, w.alignment, inp.x_bytes())
    assert run.status() == 0
    wts = W.make_topk_weights(w, inp.topk_idx)
    slots = run.layout.expert_slot.cpu().numpy().reshape(inp.topk_idx.shape)
    recv = run.rows.recv_x.view(torch.bfloat16)
    got = _run_combine(slots, wts, recv)
    x_bits = inp.x.view(torch.int16).numpy().view(np.uint16)
    x = _bf16_bits_to_f64(x_bits)
    s = x * wts.astype(np.float64).sum(axis=1, keepdims=True)
    err = (w.num_topk + 1) * U * np.abs(x) * np.abs(wts.astype(np.float64)).sum(axis=1, keepdims=True)
    g = _bf16_bits_to_f64(got)
    assert np.all(np.abs(g - s) <= 2.0 ** -8 * (np.maximum(np.abs(g), np.abs(s)) + err) + err + 2.0 ** -133)


def test_combine_full_size_workload():
    """The 4096 x 7168 top-8-of-256 batch at full size, every output checked."""
    w = W.get(W.METRIC_WORKLOAD)
    _banner(f"full size {w.describe()}")
    topk = W.make_topk(w)
    ref = oracle.layout(topk, w.num_experts, w.num_ranks, w.alignment)
    y = W.make_expert_out(w, ref.num_recv_rows)
    wts = W.make_topk_weights(w, topk)
    got = _run_combine(ref.expert_slot, wts, y)
    frac = _check(got, y.view(torch.int16).numpy().view(np.uint16), wts, ref.expert_slot)
    print(f"[gpu-combine] exact bf16 match fraction {frac:.6f}", flush=True)


def test_combine_drops_slots_outside_y():
    """A slot at or past expert_rows contributes nothing (never read)."""
    _banner("slots past expert_rows")
    w, topk, ref, y, wts = _combine_inputs(100, 4, 16, 64, 0.0, seed=13)
    slots = ref.expert_slot.copy()
    slots[5, 0] = y.shape[0]
    slots[6, 1] = y.shape[0] + 10 ** 6
    got = _run_combine(slots, wts, y)
    trimmed = np.where(slots >= y.shape[0], -1, slots)
    _check(got, y.view(torch.int16).numpy().view(np.uint16), wts, trimmed)


def test_combine_grid_loops_over_many_tokens():
    """150000 single-segment tokens need more wavefronts than one grid holds,
    so every wavefront takes several (token, segment) units in turn."""
    _banner("150000 tokens, grid-stride loop")
    w, topk, ref, y, wts = _combine_inputs(150000, 8, 64, 64, 0.05, seed=14)
    got = _run_combine(ref.expert_slot, wts, y)
    _check(got, y.view(torch.int16).numpy().view(np.uint16), wts, ref.expert_slot)


def test_combine_signed_weights():
    """Weights of both signs (the sum can cancel): the bound uses |w|, and most
    outputs still equal the exact sum rounded to bf16."""
    _banner("signed weights")
    w, topk, ref, y, wts = _combine_inputs(400, 8, 64, 520, 0.1, seed=15)
    sign = np.where(np.random.default_rng([15, 1]).random(wts.shape) < 0.5, -1.0, 1.0).astype(np.float32)
    signed = wts * sign
    got = _run_combine(ref.expert_slot, signed, y)
    _check(got, y.view(torch.int16).numpy().view(np.uint16), signed, ref.expert_slot, min_exact=0.98)


@pytest.mark.parametrize("seed", range(12))
def test_combine_random_problem(seed):
    """Seeded random combines: tokens, top-k, experts, hidden width, masking."""
    rng = np.random.default_rng([seed, 91])
    t = int(rng.choice([1, 33, 500, 3000]))
    k = int(rng.choice([1, 2, 5, 8, 13, 32]))
    e = int(rng.choice([32, 64, 256]))
    hidden = 8 * int(rng.choice([1, 16, 65, 300, 896]))
    mask = float(rng.choice([0.0, 0.1, 0.6]))
    _banner(f"random seed={seed} T={t} K={k} E={e} H={hidden} mask={mask}")
    w, topk, ref, y, wts = _combine_inputs(t, min(k, e), e, hidden, mask, seed=300 + seed)
    got = _run_combine(ref.expert_slot, wts, y)
    _check(got, y.view(torch.int16).numpy().view(np.uint16), wts, ref.expert_slot)


def test_combine_plan_equals_the_direct_call():
    _banner("combine plan")
    w, topk, ref, y, wts = _combine_inputs(300, 8, 64, 1024, 0.1, seed=16)
    slots_d = torch.from_numpy(np.ascontiguousarray(ref.expert_slot, dtype=np.int32)).to(H.DEVICE)
    wts_d = torch.from_numpy(np.ascontiguousarray(wts, dtype=np.float32)).to(H.DEVICE)
    y_d = y.to(H.DEVICE)
    out = torch.full((300, 1024), -123.0, dtype=torch.bfloat16, device=H.DEVICE)
    plan = M.CombinePlan(slots_d, wts_d, y_d, out)
    plan()
    plan()
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _run_combine(ref.expert_slot, wts, y))
    _check(got, y.view(torch.int16).numpy().view(np.uint16), wts, ref.expert_slot)
