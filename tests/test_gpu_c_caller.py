"""A dispatch driven from C alone, on the GPU: tests/_bin/c_dispatch_run
(built from tests/c_dispatch_run.c before any GPU run) allocates with
hipMalloc, fills every output with 0xA5 bytes and calls the C ABI on a stream
of its own, with no Python or torch in its process. Its outputs must equal the
CPU oracle's bit for bit, and nothing past the totals may be written.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W
from tests import c_programs
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

FILL32 = np.frombuffer(b"\xa5\xa5\xa5\xa5", dtype=np.int32)[0]


def _dispatch_from_c(tmp, topk, xb, sf, e, r, a, one_call):
    t, k = topk.shape
    rb, s = xb.shape[1], 0 if sf is None else sf.shape[1]
    inp, outp = os.path.join(tmp, "in.bin"), os.path.join(tmp, "out.bin")
    with open(inp, "wb") as f:
        np.array([t, k, e, r, a, rb, s, int(one_call)], dtype=np.int64).tofile(f)
        np.ascontiguousarray(topk, dtype=np.int64).tofile(f)
        np.ascontiguousarray(xb, dtype=np.uint8).tofile(f)
        if s:
            np.ascontiguousarray(sf, dtype=np.float32).tofile(f)
    if not os.path.exists(c_programs.DISPATCH_RUN):
        raise RuntimeError(f"{c_programs.DISPATCH_RUN} is missing: build it with `python -m tests.c_programs`")
    run = subprocess.run([c_programs.DISPATCH_RUN, inp, outp], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    buf = open(outp, "rb").read()
    pos = 0

    def take(dtype, n):
        nonlocal pos
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=pos)
        pos += a.nbytes
        return a

    out = {"rc": int(take(np.int32, 1)[0])}
    recv_cap, rank_cap = int(take(np.int64, 1)[0]), int(take(np.int64, 1)[0])
    out["status"] = int(take(np.int32, 1)[0])
    for name, n in (("expert_count", e), ("rank_count", r), ("expert_psum", e + 1), ("rank_psum", r + 1),
                    ("expert_slot", t * k), ("rank_slot", t * k), ("recv_src_token_idx", recv_cap),
                    ("rank_src_token_idx", rank_cap)):
        out[name] = take(np.int32, n)
    out["rank_x"] = take(np.uint8, rank_cap * rb).reshape(rank_cap, rb)
    out["rank_sf"] = take(np.uint8, rank_cap * s * 4).reshape(rank_cap, s * 4) if s else None
    out["recv_x"] = take(np.uint8, recv_cap * rb).reshape(recv_cap, rb)
    out["recv_sf"] = take(np.uint8, recv_cap * s * 4).reshape(recv_cap, s * 4) if s else None
    assert pos == len(buf)
    return out


@pytest.mark.parametrize("t,e,r,a,dtype,with_sf,hidden,one_call", [
    (1500, 64, 8, 16, "fp8", True, 512, False),   # layout and scatter calls, pads, scale factors
    (3000, 256, 8, 1, "bf16", False, 1024, False),
    (200, 256, 8, 4, "bf16", False, 256, True),   # the one call: one kernel
    (16, 256, 8, 128, "fp8", True, 256, False),   # small batch: pad wavefronts mapped to row blocks
])
def test_dispatch_from_c_matches_oracle(tmp_path, t, e, r, a, dtype, with_sf, hidden, one_call):
    print(f"\n[gpu-c-caller] T={t} E={e} R={r} A={a} {dtype}{'+sf' if with_sf else ''} H={hidden} "
          f"one_call={one_call}", flush=True)
    w = W.Workload("c_caller", t, hidden, dtype, with_sf, e, r, 8, mask_frac=0.05, alignment=a, seed=77 + t)
    inp = W.make_inputs(w)
    xb = inp.x_bytes()
    got = _dispatch_from_c(str(tmp_path), inp.topk_idx, xb, inp.x_sf, e, r, a, one_call)
    ref = oracle.layout(inp.topk_idx, e, r, a)
    assert got["rc"] == 0 and got["status"] == ref.status == 0
    for name in ("expert_count", "rank_count", "expert_psum", "rank_psum"):
        assert np.array_equal(got[name], getattr(ref, name)), name
    assert np.array_equal(got["expert_slot"], ref.expert_slot.ravel())
    assert np.array_equal(got["rank_slot"], ref.rank_slot.ravel())
    p, n_rank = ref.num_recv_rows, ref.num_rank_rows
    for name, n in (("recv_src_token_idx", p), ("rank_src_token_idx", n_rank)):
        assert np.array_equal(got[name][:n], getattr(ref, name)[:n]), name
        assert np.all(got[name][n:] == FILL32), f"{name} written past the total"
    want = oracle.scatter(ref, xb, inp.x_sf, fill=H.ROW_FILL)
    for name, n in (("rank_x", n_rank), ("recv_x", p), ("rank_sf", n_rank), ("recv_sf", p)):
        g, wv = got[name], getattr(want, name)
        if g is None:
            continue
        assert np.array_equal(g[:n], wv.view(np.uint8).reshape(n, -1)), f"{name} differs from the oracle"
        assert np.all(g[n:] == H.ROW_FILL), f"{name} written past the total"
