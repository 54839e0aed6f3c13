"""CPU pins for the combine checker used by the GPU tests and smoke().

The checker must accept what a correct kernel produces and reject plausible
mistakes. A correct result is emulated here step by step on the CPU: one
fp32 fused multiply-add per routed k in ascending order (the product of an
fp32 weight and a bf16 value is exact in float64, so float64 add then fp32
rounding is the fused operation up to a double rounding that these inputs
never hit), then one round-to-nearest-even to bf16.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from tests import gpu_harness as H


def _emulate(slots, wts, y_bits, rne=True):
    y = H.bf16_bits_to_f64(y_bits)
    acc = np.zeros((slots.shape[0], y.shape[1]), np.float32)
    for k in range(slots.shape[1]):
        s = slots[:, k]
        prod = wts[:, k].astype(np.float64)[:, None] * y[np.maximum(s, 0)]
        acc = np.where((s >= 0)[:, None], (acc.astype(np.float64) + prod).astype(np.float32), acc)
    u = acc.view(np.uint32).astype(np.uint64)
    if not rne:
        return (u >> 16).astype(np.uint16)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _case(seed, t=96, k=6, e=32, hidden=72, mask=0.15):
    w = W.Workload(f"chk{seed}", t, hidden, "bf16", False, e, 4, k, mask_frac=mask, seed=seed)
    topk = W.make_topk(w)
    lay = oracle.layout(topk, e, 4, 1)
    y = W.make_expert_out(w, lay.num_recv_rows)
    import torch
    y_bits = y.view(torch.int16).numpy().view(np.uint16)
    return lay.expert_slot, W.make_topk_weights(w, topk), y_bits


def test_rne_pins():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -8 + 2.0 ** -30, 0.0,
                  -(1.0 + 2.0 ** -8), 3.0 * 2.0 ** -100])
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x0000, 0xBF80, 0x0E40], dtype=np.uint16)
    assert np.array_equal(H.f64_to_bf16_rne(v), want)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_checker_accepts_fp32_chain(seed):
    slots, wts, y_bits = _case(seed)
    frac = H.assert_combine_close(_emulate(slots, wts, y_bits), y_bits, wts, slots)
    assert frac > 0.999


def test_checker_rejects_mistakes():
    slots, wts, y_bits = _case(4)
    good = _emulate(slots, wts, y_bits)
    mistakes = {
        "dropped last k": _emulate(slots[:, :-1], wts[:, :-1], y_bits),
        "low bit flipped": good ^ np.uint16(1),
        "truncated to bf16": _emulate(slots, wts, y_bits, rne=False),
        "weights of k swapped": _emulate(slots, wts[:, ::-1].copy(), y_bits),
        "unweighted sum": _emulate(slots, np.ones_like(wts), y_bits),
        "wrong row (slot + 1)": _emulate(np.where(slots >= 0, (slots + 1) % y_bits.shape[0], -1), wts, y_bits),
        "sign of one term": _emulate(slots, wts * np.where(np.arange(wts.shape[1]) == 0, -1, 1), y_bits),
    }
    for name, bits in mistakes.items():
        with pytest.raises(AssertionError):
            H.assert_combine_close(bits, y_bits, wts, slots)
            pytest.fail(f"checker accepted: {name}")


def test_checker_requires_zero_rows_for_unrouted_tokens():
    slots, wts, y_bits = _case(5)
    slots = slots.copy()
    slots[7] = -1
    bits = _emulate(slots, wts, y_bits)
    H.assert_combine_close(bits, y_bits, wts, slots)
    bits[7, 3] = 0x8000                     # -0 instead of +0
    with pytest.raises(AssertionError):
        H.assert_combine_close(bits, y_bits, wts, slots)
