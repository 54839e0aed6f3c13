"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented host error codes before touching the
GPU (no compute call runs here)."""

import ctypes
import os
import re

import pytest

import moe_token_dispatch_amd as M

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_dispatch.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dispatch_\w+)\s*\(", text, flags=re.M)))


def _defines():
    out = {}
    for name, val in re.findall(r"#define\s+(DISPATCH_\w+)\s+\(?(-?\d+)u?\)?", open(HEADER).read()):
        out[name] = int(val)
    return out


def test_library_exports_every_declared_symbol():
    lib = M.load_library()
    declared = _declared_functions()
    assert set(declared) == set(M.SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_binding_constants_match_header():
    d = _defines()
    assert d["DISPATCH_ABI_VERSION"] == M.dispatch_abi_version() == 6
    assert (d["DISPATCH_ERR_NULL"], d["DISPATCH_ERR_ARG"], d["DISPATCH_ERR_ALIGN"],
            d["DISPATCH_ERR_WORKSPACE"], d["DISPATCH_ERR_HIP"]) == (
        M.ERR_NULL, M.ERR_ARG, M.ERR_ALIGN, M.ERR_WORKSPACE, M.ERR_HIP)
    assert (d["DISPATCH_STATUS_BAD_EXPERT"], d["DISPATCH_STATUS_RECV_OVERFLOW"],
            d["DISPATCH_STATUS_RANK_OVERFLOW"], d["DISPATCH_STATUS_DUP_EXPERT"], d["DISPATCH_STATUS_BAD_COUNT"],
            d["DISPATCH_STATUS_TIMEOUT"]) == (
        M.STATUS_BAD_EXPERT, M.STATUS_RECV_OVERFLOW, M.STATUS_RANK_OVERFLOW, M.STATUS_DUP_EXPERT,
        M.STATUS_BAD_COUNT, M.STATUS_TIMEOUT)
    assert d["DISPATCH_DEFAULT_WAIT_LIMIT"] == M.DEFAULT_WAIT_LIMIT
    assert (d["DISPATCH_RANK_CONTIG"], d["DISPATCH_EXPERT_MAJOR"], d["DISPATCH_ZERO_PAD"],
            d["DISPATCH_ROWS_READ_AHEAD"]) == (M.RANK_CONTIG, M.EXPERT_MAJOR, M.ZERO_PAD, M.ROWS_READ_AHEAD)
    assert d["DISPATCH_MAX_TOPK"] == M.MAX_TOPK and d["DISPATCH_MAX_EXPERTS"] == M.MAX_EXPERTS
    assert d["DISPATCH_MAX_RANKS"] == M.MAX_RANKS
    assert ctypes.sizeof(M.Problem) == 64 and ctypes.sizeof(M.LayoutPtrs) == 10 * 8


def test_wait_limit_setter():
    """The in-kernel wait bound: a negative bound is refused, 0 restores the default."""
    lib = M.load_library()
    assert lib.dispatch_set_wait_limit(-1) == M.ERR_ARG
    assert lib.dispatch_set_wait_limit(5) == M.OK
    assert lib.dispatch_set_wait_limit(0) == M.OK
    with pytest.raises(M.DispatchError):
        M.dispatch_set_wait_limit(-3)


def test_strerror_covers_codes():
    for code in (0, -1, -2, -3, -4, -5):
        assert M.dispatch_strerror(code) and "unknown" not in M.dispatch_strerror(code)
    assert "unknown" in M.dispatch_strerror(-99)


def test_max_rows_and_workspace():
    p = M.make_problem(4096, 8, 256, 8, 1, row_bytes=14336)
    assert M.dispatch_max_rows(p) == (4096 * 8, 4096 * 8)
    p = M.make_problem(65536, 8, 256, 8, 128, row_bytes=7168, sf_per_token=56)
    assert M.dispatch_max_rows(p) == (65536 * 8 + 256 * 127, 65536 * 8)
    p = M.make_problem(100, 8, 64, 4, 4, row_bytes=64)
    assert M.dispatch_max_rows(p) == (800 + 64 * 3, 400)  # min(K, R) = 4 rank rows per token
    ws = M.dispatch_workspace_size(p)
    assert ws >= 256 and ws % 256 == 0
    # Workspace grows with the number of tiles and keys.
    assert M.dispatch_workspace_size(M.make_problem(1 << 20, 8, 256, 8)) > ws


BAD_PROBLEMS = [
    dict(num_tokens=-1), dict(num_topk=0), dict(num_topk=33), dict(num_experts=0),
    dict(num_experts=4097), dict(num_ranks=3), dict(num_ranks=0), dict(num_ranks=512),
    dict(num_experts=4096, num_ranks=2048),
    dict(expert_alignment=0), dict(topk_idx_bytes=2), dict(sf_per_token=-1), dict(flags=16),
    dict(recv_capacity_rows=-1), dict(reserved=1), dict(num_tokens=1 << 31),
    dict(num_tokens=1 << 28, expert_alignment=1 << 20),
    dict(num_tokens=(1 << 62) + 1),  # rejected before T * K is formed
]


@pytest.mark.parametrize("bad", BAD_PROBLEMS)
def test_bad_problem_rejected(bad):
    p = M.Problem(100, 8, 256, 8, 1, 8, 0, 64, 1000, 1000, M.ALL_OUTPUTS, 0)
    for k, v in bad.items():
        setattr(p, k, v)
    lib = M.load_library()
    size = ctypes.c_size_t(0)
    assert lib.dispatch_workspace_size(ctypes.byref(p), ctypes.byref(size)) == M.ERR_ARG
    lay = M.LayoutPtrs(*([16] * 9))
    assert lib.dispatch_layout(ctypes.byref(p), 16, ctypes.byref(lay), 256, 1 << 20, None) == M.ERR_ARG
    assert lib.dispatch_scatter(ctypes.byref(p), ctypes.byref(lay), 16, 16, 16, 16, 16, 16, None) == M.ERR_ARG


def test_host_errors_before_launch():
    """Null, alignment and workspace errors come back without any GPU work."""
    lib = M.load_library()
    p = M.Problem(100, 8, 256, 8, 1, 8, 4, 64, 1000, 1000, M.ALL_OUTPUTS, 0)
    good = M.LayoutPtrs(*([4096] * 9))
    ws_need = M.dispatch_workspace_size(p)
    call = lambda prob, topk, lay, ws, n: lib.dispatch_layout(  # noqa: E731
        ctypes.byref(prob) if prob is not None else None, topk,
        ctypes.byref(lay) if lay is not None else None, ws, n, None)
    assert call(None, 4096, good, 4096, ws_need) == M.ERR_NULL
    assert call(p, None, good, 4096, ws_need) == M.ERR_NULL
    assert call(p, 4096, None, 4096, ws_need) == M.ERR_NULL
    for i in range(9):
        lay = M.LayoutPtrs(*([4096] * 9))
        setattr(lay, M.LayoutPtrs._fields_[i][0], None)
        assert call(p, 4096, lay, 4096, ws_need) == M.ERR_NULL, i
    assert call(p, 4100, good, 4096, ws_need) == M.ERR_ALIGN  # int64 table not 8-byte aligned
    lay = M.LayoutPtrs(*([4096] * 9))
    lay.expert_slot = 4098
    assert call(p, 4096, lay, 4096, ws_need) == M.ERR_ALIGN
    lay = M.LayoutPtrs(*([4096] * 9))
    lay.expert_count_cumulative = 4098  # optional, but 4-byte aligned when given
    assert call(p, 4096, lay, 4096, ws_need) == M.ERR_ALIGN
    assert call(p, 4096, good, None, ws_need) == M.ERR_WORKSPACE
    assert call(p, 4096, good, 4096 + 64, ws_need) == M.ERR_WORKSPACE  # not 256-byte aligned
    assert call(p, 4096, good, 4096, ws_need - 1) == M.ERR_WORKSPACE

    sc = lambda prob, lay, x, sf, rx, rsf, ex, esf: lib.dispatch_scatter(  # noqa: E731
        ctypes.byref(prob), ctypes.byref(lay) if lay is not None else None, x, sf, rx, rsf, ex, esf, None)
    assert sc(p, None, 4096, 4096, 4096, 4096, 4096, 4096) == M.ERR_NULL
    assert sc(p, good, None, 4096, 4096, 4096, 4096, 4096) == M.ERR_NULL
    assert sc(p, good, 4096, None, 4096, 4096, 4096, 4096) == M.ERR_NULL  # S > 0 needs x_sf
    assert sc(p, good, 4096, 4096, None, 4096, 4096, 4096) == M.ERR_NULL
    assert sc(p, good, 4096, 4096, 4096, 4096, None, 4096) == M.ERR_NULL
    assert sc(p, good, 4104, 4096, 4096, 4096, 4096, 4096) == M.ERR_ALIGN  # x not 16-byte aligned
    assert sc(p, good, 4096, 4098, 4096, 4096, 4096, 4096) == M.ERR_ALIGN
    p2 = M.Problem(100, 8, 256, 8, 1, 8, 4, 72, 1000, 1000, M.ALL_OUTPUTS, 0)
    assert sc(p2, good, 4096, 4096, 4096, 4096, 4096, 4096) == M.ERR_ALIGN  # row_bytes % 16
    p3 = M.Problem(100, 8, 256, 8, 1, 8, 4, 0, 1000, 1000, M.ALL_OUTPUTS, 0)
    assert sc(p3, good, 4096, 4096, 4096, 4096, 4096, 4096) == M.ERR_ARG
    p3.row_bytes = 1 << 31  # one row must stay below 2 GiB
    assert sc(p3, good, 4096, 4096, 4096, 4096, 4096, 4096) == M.ERR_ARG
    # Only the selected outputs are required: with expert-major rows alone and
    # no scale factors, NULL rank buffers pass and a misaligned recv_x is caught.
    p4 = M.Problem(100, 8, 256, 8, 1, 8, 0, 64, 1000, 1000, M.EXPERT_MAJOR, 0)
    assert sc(p4, good, 4096, None, None, None, 4104, None) == M.ERR_ALIGN


def test_kernel_counts():
    """The layout: one kernel for a one-tile batch, two with the histograms
    reduced in the assign kernel, three with the column scan. The combined
    call: one kernel up to 3072 (token, k) pairs (2048 when pad rows are
    zeroed); beyond, when it reads the rows ahead (at most 160 MB) and the
    tiles can exchange their counts (up to 256 tiles of fewer than 4096
    (token, k) pairs whose exchange words fit 8192, a thread per count
    word), the
    one-launch layout and the scatter; else the layout's kernels and the
    scatter."""
    mk = M.make_problem
    assert M.dispatch_kernel_count(mk(256, 8, 256, 8, 1, row_bytes=14336)) == (1, 1)
    assert M.dispatch_kernel_count(mk(0, 8, 256, 8, 1, row_bytes=64)) == (1, 1)
    assert M.dispatch_kernel_count(mk(2048, 1, 64, 8, 1, row_bytes=48)) == (1, 1)
    assert M.dispatch_kernel_count(mk(257, 8, 256, 8, 1, row_bytes=14336)) == (2, 1)
    assert M.dispatch_kernel_count(mk(384, 8, 256, 8, 1, row_bytes=14336)) == (2, 1)
    assert M.dispatch_kernel_count(mk(385, 8, 256, 8, 1, row_bytes=14336)) == (2, 2)
    assert M.dispatch_kernel_count(mk(256, 8, 256, 8, 128, row_bytes=7168, sf_per_token=56)) == (1, 1)
    assert M.dispatch_kernel_count(mk(257, 8, 256, 8, 128, row_bytes=7168, sf_per_token=56)) == (2, 2)
    assert M.dispatch_kernel_count(mk(384, 8, 256, 8, 2, row_bytes=64)) == (2, 2)
    # Without the zero-pad flag nothing is padded, and the 3072-pair limit holds.
    assert M.dispatch_kernel_count(mk(384, 8, 256, 8, 2, row_bytes=64,
                                      flags=M.RANK_CONTIG | M.EXPERT_MAJOR)) == (2, 1)
    assert M.dispatch_kernel_count(mk(3072, 1, 64, 8, 1, row_bytes=48)) == (2, 1)
    assert M.dispatch_kernel_count(mk(4096, 8, 256, 8, 1, row_bytes=14336)) == (2, 2)
    assert M.dispatch_kernel_count(mk(16384, 8, 128, 16, 1, row_bytes=8192)) == (2, 2)
    # 470 MB of rows: no read-ahead, so the count and assign kernels.
    assert M.dispatch_kernel_count(mk(65536, 8, 256, 8, 128, row_bytes=7168, sf_per_token=56)) == (2, 3)
    # 514 tiles of 16 wavefronts x 4 chunks: past the one-launch layout's 256 tiles.
    assert M.dispatch_kernel_count(mk(257 * 1024, 8, 64, 8, 1, row_bytes=16)) == (2, 3)
    assert M.dispatch_kernel_count(mk(4096, 8, 4096, 1024, 1, row_bytes=64)) == (3, 4)
    assert M.dispatch_kernel_count(mk(80, 8, 4096, 1024, 1, row_bytes=64)) == (1, 1)
    # 5120 keys: 1024 count words per tile, more than a 5-wavefront tile's threads.
    assert M.dispatch_kernel_count(mk(300, 8, 4096, 1024, 1, row_bytes=64)) == (2, 1)
    assert M.dispatch_kernel_count(mk(3841, 8, 4096, 1024, 1, row_bytes=64)) == (3, 4)
    # Tiles of 256 tokens x 8 pairs hold 2048 pairs, of 512 tokens 4096: no
    # 12-bit count then, whatever the routing.
    assert M.dispatch_kernel_count(mk(31745, 8, 256, 8, 1, row_bytes=16)) == (2, 2)
    assert M.dispatch_kernel_count(mk(63489, 8, 256, 8, 1, row_bytes=16)) == (2, 3)
    assert M.dispatch_kernel_count(mk(260000, 1, 256, 8, 1, row_bytes=16)) == (2, 2)
    with pytest.raises(M.DispatchError):
        M.dispatch_kernel_count(M.Problem(10, 0, 8, 2, 1, 8, 0, 64, 100, 100, M.ALL_OUTPUTS, 0))


def test_layout_and_scatter_host_errors_before_launch():
    """The combined call makes both calls' checks before enqueuing anything."""
    lib = M.load_library()
    p = M.Problem(100, 8, 256, 8, 1, 8, 4, 64, 1000, 1000, M.ALL_OUTPUTS, 0)
    good = M.LayoutPtrs(*([4096] * 9))
    ws_need = M.dispatch_workspace_size(p)

    def call(prob, topk, lay, ws, n, x, sf, rx, rsf, ex, esf):
        return lib.dispatch_layout_and_scatter(ctypes.byref(prob) if prob is not None else None, topk,
                                               ctypes.byref(lay) if lay is not None else None, ws, n,
                                               x, sf, rx, rsf, ex, esf, None)

    rows = (4096, 4096, 4096, 4096, 4096, 4096)
    assert call(None, 4096, good, 4096, ws_need, *rows) == M.ERR_NULL
    assert call(p, None, good, 4096, ws_need, *rows) == M.ERR_NULL
    assert call(p, 4096, None, 4096, ws_need, *rows) == M.ERR_NULL
    assert call(p, 4096, good, None, ws_need, *rows) == M.ERR_WORKSPACE
    assert call(p, 4096, good, 4096, ws_need - 1, *rows) == M.ERR_WORKSPACE
    assert call(p, 4100, good, 4096, ws_need, *rows) == M.ERR_ALIGN
    assert call(p, 4096, good, 4096, ws_need, None, 4096, 4096, 4096, 4096, 4096) == M.ERR_NULL  # no x
    assert call(p, 4096, good, 4096, ws_need, 4096, None, 4096, 4096, 4096, 4096) == M.ERR_NULL  # S > 0
    assert call(p, 4096, good, 4096, ws_need, 4104, 4096, 4096, 4096, 4096, 4096) == M.ERR_ALIGN
    bad = M.Problem(100, 8, 256, 8, 1, 8, 4, 72, 1000, 1000, M.ALL_OUTPUTS, 0)  # row_bytes % 16
    assert call(bad, 4096, good, 4096, ws_need, *rows) == M.ERR_ALIGN
    bad.row_bytes, bad.num_topk = 64, 0
    assert call(bad, 4096, good, 4096, ws_need, *rows) == M.ERR_ARG


def test_layout_read_ahead_host_errors_before_launch():
    """The read-ahead layout makes the layout's checks and those of the rows
    it reads before enqueuing anything."""
    lib = M.load_library()
    p = M.Problem(100, 8, 256, 8, 1, 8, 4, 64, 1000, 1000, M.ALL_OUTPUTS, 0)
    good = M.LayoutPtrs(*([4096] * 9))
    ws_need = M.dispatch_workspace_size(p)

    def call(prob, topk, lay, ws, n, x, sf):
        return lib.dispatch_layout_read_ahead(ctypes.byref(prob) if prob is not None else None, topk,
                                              ctypes.byref(lay) if lay is not None else None, ws, n, x, sf, None)

    assert call(None, 4096, good, 4096, ws_need, 4096, 4096) == M.ERR_NULL
    assert call(p, None, good, 4096, ws_need, 4096, 4096) == M.ERR_NULL
    assert call(p, 4096, None, 4096, ws_need, 4096, 4096) == M.ERR_NULL
    assert call(p, 4096, good, None, ws_need, 4096, 4096) == M.ERR_WORKSPACE
    assert call(p, 4096, good, 4096, ws_need - 1, 4096, 4096) == M.ERR_WORKSPACE
    assert call(p, 4100, good, 4096, ws_need, 4096, 4096) == M.ERR_ALIGN
    assert call(p, 4096, good, 4096, ws_need, None, 4096) == M.ERR_NULL   # no rows
    assert call(p, 4096, good, 4096, ws_need, 4096, None) == M.ERR_NULL   # S > 0 needs scale factors
    assert call(p, 4096, good, 4096, ws_need, 4104, 4096) == M.ERR_ALIGN  # rows 16-byte aligned
    assert call(p, 4096, good, 4096, ws_need, 4096, 4098) == M.ERR_ALIGN  # scale factors 4-byte aligned
    bad = M.Problem(100, 8, 256, 8, 1, 8, 4, 72, 1000, 1000, M.ALL_OUTPUTS, 0)  # row_bytes % 16
    assert call(bad, 4096, good, 4096, ws_need, 4096, 4096) == M.ERR_ALIGN


def test_binding_refuses_host_tensors():
    import torch

    p = M.make_problem(4, 2, 8, 2, 1, row_bytes=16)
    with pytest.raises(ValueError):
        M.dispatch_layout(p, torch.zeros((4, 2), dtype=torch.int64), None, torch.zeros(256, dtype=torch.uint8))


def test_expand_host_errors():
    lib = M.load_library()
    assert ctypes.sizeof(M.ExpandProblem) == 56
    q = M.ExpandProblem(4, 100, 8, 256, 8, 3, 1, 8, 0, 0, 64, 1000)
    size = ctypes.c_size_t(0)
    assert lib.dispatch_expand_workspace_size(ctypes.byref(q), ctypes.byref(size)) == M.OK and size.value > 0
    cap = ctypes.c_int64(0)
    assert lib.dispatch_expand_max_rows(ctypes.byref(q), ctypes.byref(cap)) == M.OK
    assert cap.value == 4 * 100 * 8 + 32 * 0
    for field, bad in (("num_sources", 0), ("rows_per_source", -1), ("local_rank", 8), ("local_rank", -1),
                       ("num_ranks", 3), ("num_topk", 33), ("expert_alignment", 0), ("reserved", 1)):
        b = M.ExpandProblem(4, 100, 8, 256, 8, 3, 1, 8, 0, 0, 64, 1000)
        setattr(b, field, bad)
        assert lib.dispatch_expand_workspace_size(ctypes.byref(b), ctypes.byref(size)) == M.ERR_ARG, field
    expand_only = M.LayoutPtrs(4096, None, 4096, None, 4096, None, 4096, None, 4096)
    call = lambda lay, topk, counts, ws: lib.dispatch_expand_layout(  # noqa: E731
        ctypes.byref(q), topk, counts, ctypes.byref(lay), ws, 1 << 20, None)
    assert call(expand_only, 4096, None, 4096) == M.ERR_NULL            # recv_count required
    assert call(expand_only, None, 4096, 4096) == M.ERR_NULL            # table required when S*M > 0
    assert call(M.LayoutPtrs(*([4096] * 9)), 4096, 4096, 4096) == M.ERR_ARG  # rank outputs must be NULL
    assert call(expand_only, 4100, 4096, 4096) == M.ERR_ALIGN
    assert call(expand_only, 4096, 4096, None) == M.ERR_WORKSPACE
    assert lib.dispatch_expand_scatter(ctypes.byref(q), ctypes.byref(M.LayoutPtrs(*([4096] * 9))),
                                       4096, None, 4096, None, None) == M.ERR_ARG
    # The one-call form makes both calls' checks.
    both = lambda lay, topk, counts, ws, buf, rx: lib.dispatch_expand_layout_and_scatter(  # noqa: E731
        ctypes.byref(q), topk, counts, ctypes.byref(lay), ws, 1 << 20, buf, None, rx, None, None)
    assert both(expand_only, 4096, None, 4096, 4096, 4096) == M.ERR_NULL
    assert both(M.LayoutPtrs(*([4096] * 9)), 4096, 4096, 4096, 4096, 4096) == M.ERR_ARG
    assert both(expand_only, 4096, 4096, None, 4096, 4096) == M.ERR_WORKSPACE
    assert both(expand_only, 4096, 4096, 4096, None, 4096) == M.ERR_NULL   # received rows required
    assert both(expand_only, 4096, 4096, 4096, 4104, 4096) == M.ERR_ALIGN  # rows 16-byte aligned
    assert both(expand_only, 4096, 4096, 4096, 4096, None) == M.ERR_NULL   # expert-major output required


def test_combine_host_errors():
    lib = M.load_library()
    assert ctypes.sizeof(M.CombineProblem) == 32
    good = dict(num_tokens=4, num_topk=8, reserved=0, hidden=7168, expert_rows=64)
    call = lambda q, slot=4096, w=4096, y=4096, out=4096: lib.dispatch_combine(  # noqa: E731
        ctypes.byref(q), slot, w, y, out, None)
    for field, bad in (("num_tokens", -1), ("num_topk", 0), ("num_topk", 33), ("reserved", 1),
                       ("hidden", 0), ("hidden", 1 << 30), ("expert_rows", -1)):
        q = M.CombineProblem(**good)
        setattr(q, field, bad)
        assert call(q) == M.ERR_ARG, field
    q = M.CombineProblem(**good)
    q.hidden = 7164
    assert call(q) == M.ERR_ALIGN                       # rows must be whole 16-byte vectors
    q = M.CombineProblem(**good)
    assert call(q, slot=None) == M.ERR_NULL
    assert call(q, w=None) == M.ERR_NULL
    assert call(q, y=None) == M.ERR_NULL
    assert call(q, out=None) == M.ERR_NULL
    assert call(q, y=4104) == M.ERR_ALIGN
    assert call(q, out=4104) == M.ERR_ALIGN
    assert call(q, slot=4098) == M.ERR_ALIGN
    assert lib.dispatch_combine(None, 4096, 4096, 4096, 4096, None) == M.ERR_NULL
    empty = M.CombineProblem(**dict(good, num_tokens=0))
    assert call(empty, None, None, None, None) == M.OK  # nothing to do, nothing launched


def test_plans_keep_their_own_problem(monkeypatch):
    """A plan checks its tensors against the problem once; a later change to
    the caller's struct must not reach its C calls (host tensors stand in for
    device ones here: nothing is launched)."""
    import torch

    from moe_token_dispatch_amd import _binding as B

    monkeypatch.setattr(B, "_check_device_tensor", lambda t, name, dtype=None: None)
    monkeypatch.setattr(B, "_stream_handle", lambda stream, device: ctypes.c_void_p(0))
    p = M.make_problem(64, 8, 256, 8, 1, row_bytes=256)
    i32 = lambda n: torch.zeros(max(n, 1), dtype=torch.int32)  # noqa: E731
    lay = M.LayoutTensors(i32(256), i32(8), i32(257), i32(9), i32(512), i32(512),
                          i32(p.recv_capacity_rows), i32(p.rank_capacity_rows), i32(1))
    topk = torch.zeros((64, 8), dtype=torch.int64)
    ws = torch.zeros(M.dispatch_workspace_size(p), dtype=torch.uint8)
    x = torch.zeros((64, 256), dtype=torch.uint8)
    rows = M.RowBuffers(rank_x=torch.zeros((p.rank_capacity_rows, 256), dtype=torch.uint8), rank_sf=None,
                        recv_x=torch.zeros((p.recv_capacity_rows, 256), dtype=torch.uint8), recv_sf=None)
    plan = M.Plan(p, topk, lay, ws, x, None, rows)
    p.num_tokens = 1 << 20
    p.recv_capacity_rows = 1 << 30
    for args in (plan._layout_args, plan._scatter_args, plan._both_args):
        q = args[0]._obj
        assert q is plan._problem and q is not p
        assert q.num_tokens == 64 and q.recv_capacity_rows == 64 * 8


def test_expand_plan_keeps_its_own_problem(monkeypatch):
    import torch

    from moe_token_dispatch_amd import _binding as B

    monkeypatch.setattr(B, "_check_device_tensor", lambda t, name, dtype=None: None)
    monkeypatch.setattr(B, "_stream_handle", lambda stream, device: ctypes.c_void_p(0))
    q = M.make_expand_problem(4, 16, 8, 256, 8, 0, row_bytes=256)
    cap = q.recv_capacity_rows
    i32 = lambda n: torch.zeros(max(n, 1), dtype=torch.int32)  # noqa: E731
    lay = M.ExpandLayoutTensors(i32(32), i32(33), i32(64 * 8), i32(cap), i32(1))
    plan = M.ExpandPlan(q, torch.zeros((64, 8), dtype=torch.int64), i32(4), lay,
                        torch.zeros(M.dispatch_expand_workspace_size(q), dtype=torch.uint8),
                        torch.zeros((64, 256), dtype=torch.uint8), None,
                        torch.zeros((cap, 256), dtype=torch.uint8), None)
    q.rows_per_source = 1 << 20
    for args in (plan._layout_args, plan._scatter_args, plan._both_args):
        assert args[0]._obj is plan._problem and plan._problem.rows_per_source == 16


def test_noalloc_host_errors_before_launch():
    """The allocation-free call refuses a problem whose workspace exceeds its
    fixed device array, and a NULL problem, before anything is enqueued."""
    lib = M.load_library()
    good = M.LayoutPtrs(*([4096] * 9))
    call = lambda prob: lib.dispatch_layout_and_scatter_noalloc(  # noqa: E731
        ctypes.byref(prob) if prob is not None else None, 4096, ctypes.byref(good), 4096, 4096, 4096, 4096,
        4096, 4096, None)
    big = M.make_problem(200000, 8, 4096, 1024, 1, row_bytes=16)
    assert M.dispatch_workspace_size(big) > 4194304
    assert call(big) == M.ERR_WORKSPACE
    assert call(None) == M.ERR_NULL
    bad = M.make_problem(100, 8, 256, 8, 1, row_bytes=16)
    bad.num_topk = 0
    assert call(bad) == M.ERR_ARG


def test_read_ahead_hint_flag_is_accepted_and_other_bits_refused():
    """DISPATCH_ROWS_READ_AHEAD passes the problem check of every call (the
    layout calls ignore it); an unknown flag bit is refused."""
    p = M.make_problem(100, 8, 256, 8, 1, row_bytes=64, flags=M.ALL_OUTPUTS | M.ROWS_READ_AHEAD)
    assert M.dispatch_workspace_size(p) == M.dispatch_workspace_size(M.make_problem(100, 8, 256, 8, 1, row_bytes=64))
    assert M.dispatch_max_rows(p) == (800, 800)
    p.flags = M.ALL_OUTPUTS | 16
    with pytest.raises(M.DispatchError) as e:
        M.dispatch_workspace_size(p)
    assert e.value.code == M.ERR_ARG


def test_scatter_grid_beyond_one_launch_is_refused_before_any_launch():
    """A scatter whose grid would exceed one launch (2^32 work-items: here 64
    tokens of 2 GiB rows, 2^21 one-KB segments each) is refused with
    DISPATCH_ERR_ARG by the scatter and by the combined call, which makes the
    check before it enqueues the layout kernels."""
    lib = M.load_library()
    row = (1 << 31) - 16
    p = M.make_problem(64, 1, 8, 2, 1, 8, row, 0, 64, 64, M.ALL_OUTPUTS)
    good = M.LayoutPtrs(*([4096] * 9))
    assert lib.dispatch_scatter(ctypes.byref(p), ctypes.byref(good), 4096, None, 4096, None, 4096, None,
                                None) == M.ERR_ARG
    assert lib.dispatch_layout_and_scatter(ctypes.byref(p), 4096, ctypes.byref(good), 4096,
                                           M.dispatch_workspace_size(p), 4096, None, 4096, None, 4096, None,
                                           None) == M.ERR_ARG
    # Half the tokens fit one launch: the checks pass (nothing is launched
    # here, the NULL status pointer stops the call first).
    p.num_tokens = 16
    assert lib.dispatch_scatter(ctypes.byref(p), ctypes.byref(M.LayoutPtrs(*([4096] * 8), None)), 4096, None,
                                4096, None, 4096, None, None) == M.ERR_NULL
