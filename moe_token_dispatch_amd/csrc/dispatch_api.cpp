// C ABI of the dispatch library: argument checks, workspace sizing and the
// launches. Every check runs on the host before anything is enqueued, so a
// rejected call leaves the stream and all buffers untouched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "dispatch_common.hpp"
#include "moe_dispatch.h"

using moe_dispatch::TileGeometry;

namespace {

std::atomic<int64_t> g_wait_limit{DISPATCH_DEFAULT_WAIT_LIMIT};

bool aligned_to(const void* ptr, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(ptr) % bytes) == 0; }

// Checks shared by every entry point that takes a problem.
int check_problem(const dispatch_problem_t* p) {
    if (p == nullptr) return DISPATCH_ERR_NULL;
    if (p->num_tokens < 0) return DISPATCH_ERR_ARG;
    if (p->num_topk < 1 || p->num_topk > DISPATCH_MAX_TOPK) return DISPATCH_ERR_ARG;
    if (p->num_experts < 1 || p->num_experts > DISPATCH_MAX_EXPERTS) return DISPATCH_ERR_ARG;
    if (p->num_ranks < 1 || p->num_ranks > DISPATCH_MAX_RANKS || p->num_ranks > p->num_experts ||
        p->num_experts % p->num_ranks != 0)
        return DISPATCH_ERR_ARG;
    if (p->expert_alignment < 1) return DISPATCH_ERR_ARG;
    if (p->topk_idx_bytes != 4 && p->topk_idx_bytes != 8) return DISPATCH_ERR_ARG;
    if (p->sf_per_token < 0) return DISPATCH_ERR_ARG;
    if (p->recv_capacity_rows < 0 || p->rank_capacity_rows < 0) return DISPATCH_ERR_ARG;
    if ((p->flags & ~uint32_t(DISPATCH_ALL_OUTPUTS | DISPATCH_ROWS_READ_AHEAD)) != 0 || p->reserved != 0)
        return DISPATCH_ERR_ARG;
    // Slots and row counts are int32: the worst case must fit (T is bounded
    // first, so the product below cannot overflow).
    if (p->num_tokens > INT32_MAX) return DISPATCH_ERR_ARG;
    const int64_t worst = p->num_tokens * p->num_topk + int64_t(p->num_experts) * (p->expert_alignment - 1);
    if (worst > INT32_MAX) return DISPATCH_ERR_ARG;
    return DISPATCH_OK;
}

// The receiver-side expand runs the dispatch kernels on the receive buffer
// seen as a batch of S*M rows over the E/R local experts and a single rank.
int check_expand(const dispatch_expand_problem_t* q, dispatch_problem_t* p) {
    if (q == nullptr) return DISPATCH_ERR_NULL;
    if (q->num_sources < 1 || q->rows_per_source < 0 || q->reserved != 0) return DISPATCH_ERR_ARG;
    if (q->num_ranks < 1 || q->num_ranks > DISPATCH_MAX_RANKS || q->num_experts < 1 ||
        q->num_experts > DISPATCH_MAX_EXPERTS || q->num_experts % q->num_ranks != 0)
        return DISPATCH_ERR_ARG;
    if (q->local_rank < 0 || q->local_rank >= q->num_ranks) return DISPATCH_ERR_ARG;
    *p = dispatch_problem_t{};
    p->num_tokens = int64_t(q->num_sources) * q->rows_per_source;
    p->num_topk = q->num_topk;
    p->num_experts = q->num_experts / q->num_ranks;
    p->num_ranks = 1;
    p->expert_alignment = q->expert_alignment;
    p->topk_idx_bytes = q->topk_idx_bytes;
    p->sf_per_token = q->sf_per_token;
    p->row_bytes = q->row_bytes;
    p->recv_capacity_rows = q->recv_capacity_rows;
    p->rank_capacity_rows = INT64_MAX;  // no rank outputs; never an overflow
    p->flags = DISPATCH_EXPERT_MAJOR | DISPATCH_ZERO_PAD;
    p->reserved = 0;
    return check_problem(p);
}

// Host checks of a row scatter's arguments (the problem already checked).
int check_scatter_args(const dispatch_problem_t& p, const dispatch_layout_t* layout, const void* x,
                       const float* x_sf, void* rank_x, float* rank_sf, void* recv_x, float* recv_sf,
                       bool few_destinations) {
    if (p.row_bytes <= 0 || p.row_bytes > INT32_MAX) return DISPATCH_ERR_ARG;
    if (p.row_bytes % 16 != 0) return DISPATCH_ERR_ALIGN;
    if (layout == nullptr || !layout->status || !layout->expert_count || !layout->expert_psum)
        return DISPATCH_ERR_NULL;
    const bool want_rank = (p.flags & DISPATCH_RANK_CONTIG) != 0;
    const bool want_expert = (p.flags & DISPATCH_EXPERT_MAJOR) != 0;
    const bool want_sf = p.sf_per_token > 0;
    if (p.num_tokens > 0) {
        if (!x || !layout->expert_slot || (want_rank && !layout->rank_slot)) return DISPATCH_ERR_NULL;
        if (want_sf && !x_sf) return DISPATCH_ERR_NULL;
    }
    if (want_rank && p.rank_capacity_rows > 0 && (!rank_x || (want_sf && !rank_sf))) return DISPATCH_ERR_NULL;
    if (want_expert && p.recv_capacity_rows > 0 && (!recv_x || (want_sf && !recv_sf))) return DISPATCH_ERR_NULL;
    const void* rows[] = {x, rank_x, recv_x};
    for (const void* q : rows)
        if (q && !aligned_to(q, 16)) return DISPATCH_ERR_ALIGN;
    const void* words[] = {x_sf, rank_sf, recv_sf, layout->expert_slot, layout->rank_slot,
                           layout->expert_count, layout->expert_psum, layout->status};
    for (const void* q : words)
        if (q && !aligned_to(q, 4)) return DISPATCH_ERR_ALIGN;
    // A grid beyond one launch is refused here, before any kernel of the call.
    if (!moe_dispatch::scatter_grid_fits(p, few_destinations)) return DISPATCH_ERR_ARG;
    return DISPATCH_OK;
}

// Host checks and launch of the row scatter. few_destinations: rows go to
// about one destination each (the receiver-side expand, a top-1 expert copy).
int scatter_checked(const dispatch_problem_t* problem, const dispatch_layout_t* layout, const void* x,
                    const float* x_sf, void* rank_x, float* rank_sf, void* recv_x, float* recv_sf,
                    hipStream_t stream, bool few_destinations) {
    int rc = check_problem(problem);
    if (rc != DISPATCH_OK) return rc;
    rc = check_scatter_args(*problem, layout, x, x_sf, rank_x, rank_sf, recv_x, recv_sf, few_destinations);
    if (rc != DISPATCH_OK) return rc;
    if (moe_dispatch::launch_scatter(*problem, *layout, x, x_sf, rank_x, rank_sf, recv_x, recv_sf, stream,
                                     few_destinations) != hipSuccess)
        return DISPATCH_ERR_HIP;
    return DISPATCH_OK;
}

// Destinations per loaded row of a dispatch: K expert rows and one rank row
// at most.
bool has_few_destinations(const dispatch_problem_t& p) {
    const int experts = (p.flags & DISPATCH_EXPERT_MAJOR) ? p.num_topk : 0;
    const int ranks = (p.flags & DISPATCH_RANK_CONTIG) ? 1 : 0;
    return experts + ranks <= 1;
}

// Host checks of a layout call's arguments; on success *g is its geometry.
int check_layout_args(const dispatch_problem_t* problem, const void* topk_idx, const dispatch_layout_t* out,
                      void* workspace, size_t workspace_bytes, TileGeometry* g) {
    int rc = check_problem(problem);
    if (rc != DISPATCH_OK) return rc;
    const dispatch_problem_t& p = *problem;
    if (out == nullptr) return DISPATCH_ERR_NULL;
    if (!out->expert_count || !out->rank_count || !out->expert_psum || !out->rank_psum || !out->status)
        return DISPATCH_ERR_NULL;
    if (p.num_tokens > 0 && (!topk_idx || !out->expert_slot || !out->rank_slot)) return DISPATCH_ERR_NULL;
    if (p.recv_capacity_rows > 0 && !out->recv_src_token_idx) return DISPATCH_ERR_NULL;
    if (p.rank_capacity_rows > 0 && !out->rank_src_token_idx) return DISPATCH_ERR_NULL;
    if (workspace == nullptr) return DISPATCH_ERR_WORKSPACE;

    if (topk_idx && !aligned_to(topk_idx, p.topk_idx_bytes)) return DISPATCH_ERR_ALIGN;
    const void* ints[] = {out->expert_count, out->rank_count, out->expert_psum, out->rank_psum,
                          out->expert_slot, out->rank_slot, out->recv_src_token_idx,
                          out->rank_src_token_idx, out->status, out->expert_count_cumulative};
    for (const void* q : ints)
        if (q && !aligned_to(q, 4)) return DISPATCH_ERR_ALIGN;
    if (!aligned_to(workspace, 256)) return DISPATCH_ERR_WORKSPACE;

    *g = moe_dispatch::make_geometry(p.num_tokens, p.num_topk, p.num_experts, p.num_ranks);
    if (workspace_bytes < moe_dispatch::workspace_bytes(*g)) return DISPATCH_ERR_WORKSPACE;
    return DISPATCH_OK;
}

// Host checks of an expand layout call's arguments; on success *p is the
// dispatch problem the expand runs as, *g its geometry and *view the
// receive-buffer view.
int check_expand_layout_args(const dispatch_expand_problem_t* problem, const void* recv_topk_idx,
                             const int32_t* recv_count, const dispatch_layout_t* out, void* workspace,
                             size_t workspace_bytes, dispatch_problem_t* p, TileGeometry* g,
                             moe_dispatch::ExpandView* view) {
    int rc = check_expand(problem, p);
    if (rc != DISPATCH_OK) return rc;
    if (out == nullptr || !out->expert_count || !out->expert_psum || !out->status) return DISPATCH_ERR_NULL;
    if (out->rank_count || out->rank_psum || out->rank_slot || out->rank_src_token_idx) return DISPATCH_ERR_ARG;
    if (p->num_tokens > 0 && (!recv_topk_idx || !out->expert_slot)) return DISPATCH_ERR_NULL;
    if (!recv_count) return DISPATCH_ERR_NULL;
    if (p->recv_capacity_rows > 0 && !out->recv_src_token_idx) return DISPATCH_ERR_NULL;
    if (workspace == nullptr) return DISPATCH_ERR_WORKSPACE;
    if (recv_topk_idx && !aligned_to(recv_topk_idx, p->topk_idx_bytes)) return DISPATCH_ERR_ALIGN;
    const void* ints[] = {recv_count, out->expert_count, out->expert_psum, out->expert_slot,
                          out->recv_src_token_idx, out->status, out->expert_count_cumulative};
    for (const void* q : ints)
        if (q && !aligned_to(q, 4)) return DISPATCH_ERR_ALIGN;
    if (!aligned_to(workspace, 256)) return DISPATCH_ERR_WORKSPACE;
    *g = moe_dispatch::make_geometry(p->num_tokens, p->num_topk, p->num_experts, p->num_ranks);
    if (workspace_bytes < moe_dispatch::workspace_bytes(*g)) return DISPATCH_ERR_WORKSPACE;
    view->recv_count = recv_count;
    view->rows_per_source = problem->rows_per_source;
    view->first_expert = problem->local_rank * (problem->num_experts / problem->num_ranks);
    view->global_experts = problem->num_experts;
    return DISPATCH_OK;
}

}  // namespace

int64_t moe_dispatch::exchange_wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }

extern "C" {

int dispatch_abi_version(void) { return DISPATCH_ABI_VERSION; }

int dispatch_set_wait_limit(int64_t polls) {
    if (polls < 0) return DISPATCH_ERR_ARG;
    g_wait_limit.store(polls == 0 ? DISPATCH_DEFAULT_WAIT_LIMIT : polls, std::memory_order_relaxed);
    return DISPATCH_OK;
}

const char* dispatch_strerror(int code) {
    switch (code) {
        case DISPATCH_OK: return "success";
        case DISPATCH_ERR_NULL: return "a required pointer is NULL";
        case DISPATCH_ERR_ARG: return "a size, count or flag is out of range";
        case DISPATCH_ERR_ALIGN: return "row_bytes is not a multiple of 16 or a pointer is misaligned";
        case DISPATCH_ERR_WORKSPACE: return "workspace is missing, too small or not 256-byte aligned";
        case DISPATCH_ERR_HIP: return "the HIP runtime refused a kernel launch";
        default: return "unknown dispatch error code";
    }
}

int dispatch_workspace_size(const dispatch_problem_t* problem, size_t* bytes) {
    int rc = check_problem(problem);
    if (rc != DISPATCH_OK) return rc;
    if (bytes == nullptr) return DISPATCH_ERR_NULL;
    const TileGeometry g = moe_dispatch::make_geometry(problem->num_tokens, problem->num_topk,
                                                       problem->num_experts, problem->num_ranks);
    *bytes = moe_dispatch::workspace_bytes(g);
    return DISPATCH_OK;
}

int dispatch_max_rows(const dispatch_problem_t* problem, int64_t* max_recv_rows, int64_t* max_rank_rows) {
    int rc = check_problem(problem);
    if (rc != DISPATCH_OK) return rc;
    const int64_t k_or_r = problem->num_topk < problem->num_ranks ? problem->num_topk : problem->num_ranks;
    if (max_recv_rows)
        *max_recv_rows = problem->num_tokens * problem->num_topk +
                         int64_t(problem->num_experts) * (problem->expert_alignment - 1);
    if (max_rank_rows) *max_rank_rows = problem->num_tokens * k_or_r;
    return DISPATCH_OK;
}

int dispatch_layout(const dispatch_problem_t* problem, const void* topk_idx, const dispatch_layout_t* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    TileGeometry g;
    const int rc = check_layout_args(problem, topk_idx, out, workspace, workspace_bytes, &g);
    if (rc != DISPATCH_OK) return rc;
    if (moe_dispatch::launch_layout(*problem, g, topk_idx, *out, workspace, stream) != hipSuccess)
        return DISPATCH_ERR_HIP;
    return DISPATCH_OK;
}

int dispatch_layout_read_ahead(const dispatch_problem_t* problem, const void* topk_idx, const dispatch_layout_t* out,
                               void* workspace, size_t workspace_bytes, const void* x, const float* x_sf,
                               hipStream_t stream) {
    TileGeometry g;
    const int rc = check_layout_args(problem, topk_idx, out, workspace, workspace_bytes, &g);
    if (rc != DISPATCH_OK) return rc;
    const dispatch_problem_t& p = *problem;
    if (p.num_tokens > 0 && p.row_bytes > 0 && x == nullptr) return DISPATCH_ERR_NULL;
    if (p.num_tokens > 0 && p.sf_per_token > 0 && x_sf == nullptr) return DISPATCH_ERR_NULL;
    if (p.row_bytes < 0 || p.row_bytes % 16 != 0 || (x && !aligned_to(x, 16)) || (x_sf && !aligned_to(x_sf, 4)))
        return DISPATCH_ERR_ALIGN;
    moe_dispatch::ReadAhead ra{x, p.num_tokens * p.row_bytes, x_sf, p.num_tokens * p.sf_per_token};
    const bool read_ahead = moe_dispatch::read_ahead_fits(ra.x_bytes, ra.sf_words);
    const hipError_t err =
        read_ahead && moe_dispatch::exchange_layout_fits(p, g)
            ? moe_dispatch::launch_exchange_layout(p, g, topk_idx, *out, workspace, &ra, stream)
            : moe_dispatch::launch_layout(p, g, topk_idx, *out, workspace, stream, nullptr, read_ahead ? &ra : nullptr);
    return err == hipSuccess ? DISPATCH_OK : DISPATCH_ERR_HIP;
}

int dispatch_kernel_count(const dispatch_problem_t* problem, int* layout_kernels, int* layout_and_scatter_kernels) {
    const int rc = check_problem(problem);
    if (rc != DISPATCH_OK) return rc;
    const TileGeometry g = moe_dispatch::make_geometry(problem->num_tokens, problem->num_topk,
                                                       problem->num_experts, problem->num_ranks);
    const int layout = g.num_tiles == 1 && !g.column_scan ? 1 : (g.column_scan ? 3 : 2);
    if (layout_kernels) *layout_kernels = layout;
    // The combined call lays out in one launch when it reads the rows ahead
    // and the tiles can exchange their counts.
    const bool read_ahead = moe_dispatch::read_ahead_fits(problem->num_tokens * problem->row_bytes,
                                                          problem->num_tokens * problem->sf_per_token);
    const bool exchange = read_ahead && moe_dispatch::exchange_layout_fits(*problem, g);
    if (layout_and_scatter_kernels)
        *layout_and_scatter_kernels = moe_dispatch::fused_shape(*problem, g).fits ? 1 : (exchange ? 1 : layout) + 1;
    return DISPATCH_OK;
}

int dispatch_layout_and_scatter(const dispatch_problem_t* problem, const void* topk_idx,
                                const dispatch_layout_t* out, void* workspace, size_t workspace_bytes,
                                const void* x, const float* x_sf, void* rank_x, float* rank_sf, void* recv_x,
                                float* recv_sf, hipStream_t stream) {
    TileGeometry g;
    int rc = check_layout_args(problem, topk_idx, out, workspace, workspace_bytes, &g);
    if (rc != DISPATCH_OK) return rc;
    rc = check_scatter_args(*problem, out, x, x_sf, rank_x, rank_sf, recv_x, recv_sf,
                            has_few_destinations(*problem));
    if (rc != DISPATCH_OK) return rc;
    const dispatch_problem_t& p = *problem;
    if (moe_dispatch::fused_shape(p, g).fits) {
        if (moe_dispatch::launch_fused_dispatch(p, g, topk_idx, *out, workspace, x, x_sf, rank_x, rank_sf, recv_x,
                                                recv_sf, stream) != hipSuccess)
            return DISPATCH_ERR_HIP;
        return DISPATCH_OK;
    }
    // The layout kernels read the token rows ahead for the scatter when the
    // batch fits the Infinity Cache, and the scatter then runs as after
    // dispatch_layout_read_ahead.
    moe_dispatch::ReadAhead ra{x, p.num_tokens * p.row_bytes, x_sf, p.num_tokens * p.sf_per_token};
    const bool read_ahead = moe_dispatch::read_ahead_fits(ra.x_bytes, ra.sf_words);
    dispatch_problem_t sp = p;
    if (read_ahead) sp.flags |= DISPATCH_ROWS_READ_AHEAD;
    const bool exchange = read_ahead && moe_dispatch::exchange_layout_fits(p, g);
    if ((exchange ? moe_dispatch::launch_exchange_layout(p, g, topk_idx, *out, workspace, &ra, stream)
                  : moe_dispatch::launch_layout(p, g, topk_idx, *out, workspace, stream, nullptr,
                                                read_ahead ? &ra : nullptr)) != hipSuccess ||
        moe_dispatch::launch_scatter(sp, *out, x, x_sf, rank_x, rank_sf, recv_x, recv_sf, stream,
                                     has_few_destinations(p)) != hipSuccess)
        return DISPATCH_ERR_HIP;
    return DISPATCH_OK;
}


int dispatch_scatter(const dispatch_problem_t* problem, const dispatch_layout_t* layout, const void* x,
                     const float* x_sf, void* rank_x, float* rank_sf, void* recv_x, float* recv_sf,
                     hipStream_t stream) {
    const bool few = problem != nullptr && has_few_destinations(*problem);
    return scatter_checked(problem, layout, x, x_sf, rank_x, rank_sf, recv_x, recv_sf, stream, few);
}

int dispatch_expand_workspace_size(const dispatch_expand_problem_t* problem, size_t* bytes) {
    dispatch_problem_t p;
    int rc = check_expand(problem, &p);
    if (rc != DISPATCH_OK) return rc;
    return dispatch_workspace_size(&p, bytes);
}

int dispatch_expand_max_rows(const dispatch_expand_problem_t* problem, int64_t* max_recv_rows) {
    dispatch_problem_t p;
    int rc = check_expand(problem, &p);
    if (rc != DISPATCH_OK) return rc;
    if (max_recv_rows) {
        const int64_t k = p.num_topk < p.num_experts ? p.num_topk : p.num_experts;
        *max_recv_rows = p.num_tokens * k + int64_t(p.num_experts) * (p.expert_alignment - 1);
    }
    return DISPATCH_OK;
}

int dispatch_expand_layout(const dispatch_expand_problem_t* problem, const void* recv_topk_idx,
                           const int32_t* recv_count, const dispatch_layout_t* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    dispatch_problem_t p;
    TileGeometry g;
    moe_dispatch::ExpandView view;
    const int rc = check_expand_layout_args(problem, recv_topk_idx, recv_count, out, workspace, workspace_bytes,
                                            &p, &g, &view);
    if (rc != DISPATCH_OK) return rc;
    if (moe_dispatch::launch_layout(p, g, recv_topk_idx, *out, workspace, stream, &view) != hipSuccess)
        return DISPATCH_ERR_HIP;
    return DISPATCH_OK;
}

int dispatch_expand_layout_and_scatter(const dispatch_expand_problem_t* problem, const void* recv_topk_idx,
                                       const int32_t* recv_count, const dispatch_layout_t* out, void* workspace,
                                       size_t workspace_bytes, const void* recv_buf, const float* recv_sf_buf,
                                       void* recv_x, float* recv_sf, hipStream_t stream) {
    dispatch_problem_t p;
    TileGeometry g;
    moe_dispatch::ExpandView view;
    int rc = check_expand_layout_args(problem, recv_topk_idx, recv_count, out, workspace, workspace_bytes, &p, &g,
                                      &view);
    if (rc != DISPATCH_OK) return rc;
    rc = check_scatter_args(p, out, recv_buf, recv_sf_buf, nullptr, nullptr, recv_x, recv_sf, true);
    if (rc != DISPATCH_OK) return rc;
    if (moe_dispatch::fused_shape(p, g, true).fits) {
        if (moe_dispatch::launch_fused_dispatch(p, g, recv_topk_idx, *out, workspace, recv_buf, recv_sf_buf, nullptr,
                                                nullptr, recv_x, recv_sf, stream, &view) != hipSuccess)
            return DISPATCH_ERR_HIP;
        return DISPATCH_OK;
    }
    if (moe_dispatch::launch_layout(p, g, recv_topk_idx, *out, workspace, stream, &view) != hipSuccess ||
        moe_dispatch::launch_scatter(p, *out, recv_buf, recv_sf_buf, nullptr, nullptr, recv_x, recv_sf, stream,
                                     true) != hipSuccess)
        return DISPATCH_ERR_HIP;
    return DISPATCH_OK;
}

int dispatch_expand_scatter(const dispatch_expand_problem_t* problem, const dispatch_layout_t* layout,
                            const void* recv_buf, const float* recv_sf_buf, void* recv_x, float* recv_sf,
                            hipStream_t stream) {
    dispatch_problem_t p;
    int rc = check_expand(problem, &p);
    if (rc != DISPATCH_OK) return rc;
    if (layout != nullptr && (layout->rank_slot || layout->rank_count)) return DISPATCH_ERR_ARG;
    p.rank_capacity_rows = 0;
    return scatter_checked(&p, layout, recv_buf, recv_sf_buf, nullptr, nullptr, recv_x, recv_sf, stream, true);
}

int dispatch_combine(const dispatch_combine_problem_t* problem, const int32_t* expert_slot,
                     const float* topk_weights, const void* y, void* out, hipStream_t stream) {
    if (problem == nullptr) return DISPATCH_ERR_NULL;
    const dispatch_combine_problem_t& p = *problem;
    if (p.num_tokens < 0 || p.num_tokens > INT32_MAX || p.num_topk < 1 || p.num_topk > DISPATCH_MAX_TOPK ||
        p.reserved != 0 || p.expert_rows < 0)
        return DISPATCH_ERR_ARG;
    if (p.hidden < 8 || p.hidden > (int64_t(1) << 30) - 8) return DISPATCH_ERR_ARG;
    if (p.hidden % 8 != 0) return DISPATCH_ERR_ALIGN;
    if (p.num_tokens > 0 && (!expert_slot || !topk_weights || !out || (p.expert_rows > 0 && !y)))
        return DISPATCH_ERR_NULL;
    const void* rows[] = {y, out};
    for (const void* q : rows)
        if (q && !aligned_to(q, 16)) return DISPATCH_ERR_ALIGN;
    const void* words[] = {expert_slot, topk_weights};
    for (const void* q : words)
        if (q && !aligned_to(q, 4)) return DISPATCH_ERR_ALIGN;
    if (moe_dispatch::launch_combine(p.num_tokens, p.num_topk, p.hidden * 2, p.expert_rows, expert_slot,
                                     topk_weights, y, out, stream) != hipSuccess)
        return DISPATCH_ERR_HIP;
    return DISPATCH_OK;
}

}  // extern "C"
