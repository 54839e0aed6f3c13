"""Seeded synthetic inputs for MoE token dispatch: a token batch and a routing table.

This module only draws numbers. It holds no step of the dispatch method (no
counting, no prefix sum, no slot arithmetic), so that the CPU oracle's tests and
the HIP path's tests and benchmark can consume the same bytes without sharing
any of the method's code.

Inputs follow the problem statement of the "DeepEP Counting Sort /
Bucketization" page (section 4.2): a routing table ``topk_idx[T, K]`` of expert
ids, where a negative entry is masked, and a token batch ``x[T, H]`` in bf16 or
fp8 e4m3 with one fp32 scale factor per 128 channels.

Random streams: ``numpy.random.default_rng([seed, stream])`` (PCG64) with
stream 0 = routing noise, 1 = mask positions, 2 = x, 3 = scale factors,
4 = Zipf expert permutation, 5 = rank-locality choices, 6 = top-k weights,
7 = expert outputs (for combine).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ROUTING_UNIFORM = "uniform"      # K distinct experts, uniform over all E
ROUTING_ZIPF = "zipf"            # K distinct experts, Plackett-Luce with Zipf weights
ROUTING_RANK_LOCAL = "ranklocal"  # half uniform, half confined to 2 ranks per token
ROUTING_SINGLE = "single"        # every token picks expert 0..K-1 (all load on few experts)

_STREAM_ROUTING, _STREAM_MASK, _STREAM_X, _STREAM_SF, _STREAM_PERM, _STREAM_LOCAL, _STREAM_WEIGHTS, \
    _STREAM_EXPERT_OUT = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic dispatch problem."""

    name: str
    num_tokens: int
    hidden: int
    dtype: str                 # "bf16" or "fp8" (OCP e4m3fn)
    with_sf: bool              # fp32 scale factor per 128 channels
    num_experts: int
    num_ranks: int
    num_topk: int
    routing: str = ROUTING_UNIFORM
    zipf_s: float = 1.2
    mask_frac: float = 0.0     # exactly round(mask_frac * T * K) entries set to -1
    alignment: int = 1         # per-expert slot alignment (1 = none)
    seed: int = 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 1

    @property
    def row_bytes(self) -> int:
        return self.hidden * self.elem_bytes

    @property
    def sf_per_token(self) -> int:
        return self.hidden // 128 if self.with_sf else 0

    def describe(self) -> str:
        return (f"{self.name}: T={self.num_tokens} H={self.hidden} {self.dtype}"
                f"{'+sf' if self.with_sf else ''} E={self.num_experts} R={self.num_ranks}"
                f" K={self.num_topk} routing={self.routing} mask={self.mask_frac}"
                f" A={self.alignment}")


# The five dispatch workloads: a tiny case, the 4096 x 7168 bf16 top-8-of-256
# case the throughput metric is quoted on, its fp8 + scale-factor variant with
# 128-slot expert alignment, a heavily skewed Zipf case and a large rank-local
# fp8 case.
WORKLOADS = {
    "tiny": Workload("tiny", 256, 128, "bf16", False, 16, 4, 4, seed=1),
    "dsv3_bf16": Workload("dsv3_bf16", 4096, 7168, "bf16", False, 256, 8, 8,
                          mask_frac=0.05, seed=2),
    "dsv3_fp8_a128": Workload("dsv3_fp8_a128", 4096, 7168, "fp8", True, 256, 8, 8,
                              alignment=128, seed=3),
    "zipf_bf16": Workload("zipf_bf16", 16384, 4096, "bf16", False, 128, 16, 8,
                          routing=ROUTING_ZIPF, zipf_s=1.2, mask_frac=0.02, seed=4),
    "ranklocal_fp8_a128": Workload("ranklocal_fp8_a128", 65536, 7168, "fp8", True, 256, 8, 8,
                                   routing=ROUTING_RANK_LOCAL, alignment=128, seed=5),
}
WORKLOAD_ORDER = ["tiny", "dsv3_bf16", "dsv3_fp8_a128", "zipf_bf16", "ranklocal_fp8_a128"]
METRIC_WORKLOAD = "dsv3_bf16"


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def _gumbel_topk(rng: np.random.Generator, logits: np.ndarray, n: int, k: int,
                 chunk: int = 8192) -> np.ndarray:
    """Sample k distinct columns per row without replacement, weights exp(logits).

    Gumbel-top-k: the k largest of logits + Gumbel noise, in descending order,
    are a draw without replacement (Plackett-Luce). Zero logits give a uniform
    random k-subset in random order.
    """
    e = logits.shape[-1]
    out = np.empty((n, k), dtype=np.int64)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        g = rng.gumbel(size=(hi - lo, e)) + logits
        out[lo:hi] = np.argsort(-g, axis=1, kind="stable")[:, :k]
    return out


def make_topk(w: Workload) -> np.ndarray:
    """Routing table topk_idx[T, K] (int64); masked entries are -1."""
    t, e, r, k = w.num_tokens, w.num_experts, w.num_ranks, w.num_topk
    rng = _rng(w.seed, _STREAM_ROUTING)
    if w.routing == ROUTING_UNIFORM:
        topk = _gumbel_topk(rng, np.zeros(e), t, k)
    elif w.routing == ROUTING_ZIPF:
        perm = _rng(w.seed, _STREAM_PERM).permutation(e)
        logits = np.empty(e)
        logits[perm] = -w.zipf_s * np.log(np.arange(1, e + 1, dtype=np.float64))
        topk = _gumbel_topk(rng, logits, t, k)
    elif w.routing == ROUTING_RANK_LOCAL:
        epr = e // r
        if k > 2 * epr:
            raise ValueError("rank-local routing needs K <= 2 * experts per rank")
        lrng = _rng(w.seed, _STREAM_LOCAL)
        local = np.zeros(t, dtype=bool)
        local[lrng.permutation(t)[: t // 2]] = True
        topk = _gumbel_topk(rng, np.zeros(e), t, k)
        n_local = int(local.sum())
        if n_local:
            ranks = _gumbel_topk(lrng, np.zeros(r), n_local, 2)           # 2 distinct ranks
            cand = (ranks[:, :, None] * epr + np.arange(epr)[None, None, :]).reshape(n_local, 2 * epr)
            pick = _gumbel_topk(lrng, np.zeros(2 * epr), n_local, k)     # k distinct of those
            topk[local] = np.take_along_axis(cand, pick, axis=1)
    elif w.routing == ROUTING_SINGLE:
        topk = np.tile(np.arange(k, dtype=np.int64), (t, 1))
    else:
        raise ValueError(f"unknown routing {w.routing!r}")
    n_mask = int(round(w.mask_frac * t * k))
    if n_mask:
        flat = topk.reshape(-1)
        flat[_rng(w.seed, _STREAM_MASK).permutation(t * k)[:n_mask]] = -1
    return np.ascontiguousarray(topk)


def make_x(w: Workload, chunk_rows: int = 4096):
    """Token batch x[T, H] as a CPU torch tensor (bf16 or float8_e4m3fn), N(0,1) cast with RNE."""
    import torch

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float8_e4m3fn
    x = torch.empty((w.num_tokens, w.hidden), dtype=dt)
    rng = _rng(w.seed, _STREAM_X)
    for lo in range(0, w.num_tokens, chunk_rows):
        hi = min(w.num_tokens, lo + chunk_rows)
        x[lo:hi] = torch.from_numpy(rng.standard_normal((hi - lo, w.hidden), dtype=np.float32)).to(dt)
    return x


def make_sf(w: Workload) -> Optional[np.ndarray]:
    """Scale factors x_sf[T, H/128] (fp32, uniform in [0.5, 2]), or None."""
    if not w.with_sf:
        return None
    rng = _rng(w.seed, _STREAM_SF)
    return rng.uniform(0.5, 2.0, size=(w.num_tokens, w.sf_per_token)).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    topk_idx: np.ndarray          # int64 [T, K]
    x: object                     # torch CPU tensor [T, H]
    x_sf: Optional[np.ndarray]    # float32 [T, S] or None

    def x_bytes(self) -> np.ndarray:
        """x as raw bytes, uint8 [T, row_bytes]."""
        import torch

        return self.x.view(torch.uint8).numpy().reshape(self.workload.num_tokens, self.workload.row_bytes)


def make_inputs(w: Workload, with_x: bool = True) -> Inputs:
    x = make_x(w) if with_x else None
    return Inputs(w, make_topk(w), x, make_sf(w))


def get(name: str) -> Workload:
    return WORKLOADS[name]


def make_topk_weights(w: Workload, topk_idx: np.ndarray) -> np.ndarray:
    """Gate weights [T, K] fp32: positive, uniform in [0.1, 1], normalised (in
    float64) over each token's routed entries; masked entries get 0."""
    rng = _rng(w.seed, _STREAM_WEIGHTS)
    raw = rng.uniform(0.1, 1.0, size=topk_idx.shape)
    raw = np.where(topk_idx >= 0, raw, 0.0)
    tot = raw.sum(axis=1, keepdims=True)
    return (raw / np.where(tot > 0, tot, 1.0)).astype(np.float32)


def make_expert_out(w: Workload, rows: int):
    """Expert outputs [rows, H] as a CPU bf16 tensor, N(0,1) cast with RNE."""
    import torch

    rng = _rng(w.seed, _STREAM_EXPERT_OUT)
    y = torch.empty((rows, w.hidden), dtype=torch.bfloat16)
    for lo in range(0, rows, 4096):
        hi = min(rows, lo + 4096)
        y[lo:hi] = torch.from_numpy(rng.standard_normal((hi - lo, w.hidden), dtype=np.float32)).to(torch.bfloat16)
    return y
