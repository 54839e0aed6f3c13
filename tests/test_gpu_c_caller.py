"""The library driven from C alone, on the GPU: tests/_bin/c_dispatch_run
(built from tests/c_dispatch_run.c before any GPU run) allocates with
hipMalloc, fills every output with 0xA5 bytes and calls the C ABI on a stream
of its own, with no Python or torch in its process. The dispatch and the
receiver-side expand must equal the CPU oracle bit for bit, with nothing
written past the totals; the combine must meet its bound.
"""

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import c_programs
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

FILL32 = np.frombuffer(b"\xa5\xa5\xa5\xa5", dtype=np.int32)[0]


def _run_c(tmp, mode, arrays):
    """Writes the input arrays in order, runs the C driver, returns the output
    bytes and a reader over them."""
    inp, outp = os.path.join(tmp, f"{mode}_in.bin"), os.path.join(tmp, f"{mode}_out.bin")
    with open(inp, "wb") as f:
        for a in arrays:
            if a is not None:
                np.ascontiguousarray(a).tofile(f)
    if not os.path.exists(c_programs.DISPATCH_RUN):
        raise RuntimeError(f"{c_programs.DISPATCH_RUN} is missing: build it with `python -m tests.c_programs`")
    run = subprocess.run([c_programs.DISPATCH_RUN, mode, inp, outp], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    buf = open(outp, "rb").read()
    pos = [0]

    def take(dtype, n):
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=pos[0])
        pos[0] += a.nbytes
        return a

    def done():
        assert pos[0] == len(buf)

    return take, done


def _dispatch_from_c(tmp, topk, xb, sf, e, r, a, one_call):
    t, k = topk.shape
    rb, s = xb.shape[1], 0 if sf is None else sf.shape[1]
    take, done = _run_c(tmp, "dispatch", [
        np.array([t, k, e, r, a, rb, s, int(one_call)], dtype=np.int64), topk.astype(np.int64),
        xb.astype(np.uint8), None if sf is None else sf.astype(np.float32)])
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
    done()
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


@pytest.mark.parametrize("s_count,t,a,with_sf,one_call", [
    (4, 300, 16, True, False),   # expand layout and scatter calls
    (2, 40, 128, True, True),    # the one call
    (3, 200, 1, False, False),
])
def test_expand_from_c_matches_oracle(tmp_path, s_count, t, a, with_sf, one_call):
    from tests.test_gpu_expand import _receive_buffer, _source

    print(f"\n[gpu-c-caller] expand S={s_count} T={t} A={a} sf={with_sf} one_call={one_call}", flush=True)
    e, r, k, rank = 256, 8, 8, 5
    sources = [_source(880 + 3 * s + t, t, 512, "fp8" if with_sf else "bf16", with_sf, e, r, k, 0.05)
               for s in range(s_count)]
    recv_topk, recv_buf, recv_sf, counts, m = _receive_buffer(sources, e, r, rank, slack=4, seed=t)
    rb, sfw = recv_buf.shape[1], 0 if recv_sf is None else recv_sf.shape[1]
    take, done = _run_c(str(tmp_path), "expand", [
        np.array([s_count, m, k, e, r, rank, a, rb, sfw, int(one_call)], dtype=np.int64),
        recv_topk.astype(np.int64), counts.astype(np.int32), recv_buf, recv_sf])
    rc = int(take(np.int32, 1)[0])
    recv_cap = int(take(np.int64, 1)[0])
    status = int(take(np.int32, 1)[0])
    el = e // r
    expert_count, expert_psum = take(np.int32, el), take(np.int32, el + 1)
    expert_slot = take(np.int32, s_count * m * k)
    src = take(np.int32, recv_cap)
    recv_x = take(np.uint8, recv_cap * rb).reshape(recv_cap, rb)
    recv_sf_out = take(np.uint8, recv_cap * sfw * 4).reshape(recv_cap, sfw * 4) if sfw else None
    done()
    ref = oracle.expand_layout(recv_topk, counts, s_count, m, e, r, rank, a)
    assert rc == 0 and status == ref.status == 0
    assert np.array_equal(expert_count, ref.expert_count) and np.array_equal(expert_psum, ref.expert_psum)
    assert np.array_equal(expert_slot, ref.expert_slot.ravel())
    p = ref.num_recv_rows
    assert np.array_equal(src[:p], ref.recv_src_row_idx[:p]) and np.all(src[p:] == FILL32)
    want = oracle.expand_scatter(ref, recv_buf, recv_sf, fill=H.ROW_FILL)
    assert np.array_equal(recv_x[:p], want.recv_x) and np.all(recv_x[p:] == H.ROW_FILL)
    if sfw:
        assert np.array_equal(recv_sf_out[:p], want.recv_sf.view(np.uint8).reshape(p, -1))
        assert np.all(recv_sf_out[p:] == H.ROW_FILL)


@pytest.mark.parametrize("t,k,e,hidden,mask", [(512, 8, 256, 7168, 0.05), (257, 6, 32, 2056, 0.1)])
def test_combine_from_c_meets_its_bound(tmp_path, t, k, e, hidden, mask):
    from tests.test_gpu_combine import _combine_inputs

    print(f"\n[gpu-c-caller] combine T={t} K={k} E={e} H={hidden}", flush=True)
    w, topk, ref, y, wts = _combine_inputs(t, k, e, hidden, mask, seed=4400 + t)
    y_bits = y.view(torch.int16).numpy().view(np.uint16)
    take, done = _run_c(str(tmp_path), "combine", [
        np.array([t, k, hidden, y_bits.shape[0]], dtype=np.int64), ref.expert_slot.astype(np.int32),
        wts.astype(np.float32), y_bits])
    rc = int(take(np.int32, 1)[0])
    got = take(np.uint16, t * hidden).reshape(t, hidden)
    done()
    assert rc == 0
    H.assert_combine_close(got, y_bits, wts, ref.expert_slot)
