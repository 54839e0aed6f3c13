"""MI355X-native MoE token dispatch.

Layout (Count -> Prefix Sum -> stable slots) and row scatter of a token batch
into a rank-contiguous buffer and an expert-major buffer, as hand-written HIP
kernels for gfx950 behind a C ABI (``include/moe_dispatch.h``). This package is
the thin Python binding: it marshals torch device tensors and the current
stream into the C calls.
"""

from ._binding import (  # noqa: F401
    ALL_OUTPUTS, ERR_ALIGN, ERR_ARG, ERR_HIP, ERR_NULL, ERR_WORKSPACE, EXPERT_MAJOR, MAX_EXPERTS, Plan,
    MAX_RANKS, MAX_TOPK, OK, RANK_CONTIG, STATUS_BAD_EXPERT, STATUS_DUP_EXPERT, STATUS_RANK_OVERFLOW,
    STATUS_RECV_OVERFLOW, SYMBOLS, ZERO_PAD, DispatchError, LayoutPtrs, LayoutTensors, Problem,
    RowBuffers, alloc_layout, alloc_rows, alloc_workspace, dispatch_abi_version, dispatch_layout,
    dispatch_max_rows, dispatch_scatter, dispatch_layout_and_scatter, dispatch_kernel_count,
    dispatch_layout_read_ahead, dispatch_layout_and_scatter_noalloc, ROWS_READ_AHEAD,
    dispatch_strerror, dispatch_workspace_size, load_library, make_problem, STATUS_BAD_COUNT, ExpandProblem, ExpandLayoutTensors, make_expand_problem,
    dispatch_expand_workspace_size, alloc_expand_layout, alloc_expand_workspace, dispatch_expand_layout,
    dispatch_expand_scatter, dispatch_expand_layout_and_scatter, ExpandPlan, CombineProblem, dispatch_combine,
    CombinePlan, STATUS_TIMEOUT, DEFAULT_WAIT_LIMIT, dispatch_set_wait_limit,
)
