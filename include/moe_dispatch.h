/*
 * moe_dispatch.h: C ABI of the MI355X (gfx950) MoE token dispatch library.
 *
 * The library computes the dispatch layout of a token batch as a counting
 * sort ("DeepEP Counting Sort / Bucketization" page: Count -> Prefix Sum ->
 * Scatter, sections 2 to 8) and moves the token rows into two layouts:
 *
 *   - a rank-contiguous buffer: one row per (token, destination rank), rank r's
 *     block is rows [rank_psum[r], rank_psum[r+1]) (the page's rank-level
 *     scatter, section 6.2-6.3);
 *   - an expert-major buffer recv_x: one row per routed (token, expert) pair,
 *     expert e's bucket is rows [expert_psum[e], expert_psum[e+1]), padded with
 *     zero rows up to a multiple of the expert alignment (the page's expand
 *     mode and copy epilogue, sections 6.4, 7 and 8).
 *
 * A "rank" is a logical group of E/R consecutive experts on this one GPU:
 * expert e belongs to rank e / (E/R). Inside every expert bucket and every
 * rank block, rows follow ascending token index, so the whole layout is unique
 * and deterministic. The (token, rank) slot is held by the highest k of that
 * rank in the token (the page's dedup "master lane", section 4.2).
 *
 * Conventions for every entry point:
 *   - Ownership: all buffer pointers are device pointers allocated and owned by
 *     the caller. The library allocates, frees and retains no memory.
 *   - Asynchrony: all work is enqueued on `stream` (a hipStream_t, NULL = the
 *     null stream); no entry point synchronizes. Buffers must stay alive until
 *     the stream has passed the work.
 *   - Host errors: a negative return code is given before anything is
 *     enqueued (see DISPATCH_ERR_*).
 *   - Device errors: dispatch_layout writes a status word (DISPATCH_STATUS_*).
 *     When it is non-zero, slot maps, inverse maps and rows are unspecified and
 *     dispatch_scatter writes no row.
 *   - Rows and inverse-map entries beyond the totals (expert_psum[E],
 *     rank_psum[R]) up to the capacities are never written.
 *   - Reentrancy: concurrent calls need their own workspaces and outputs. A
 *     dispatch workspace is zero-filled once by its owner and then kept by
 *     the calls (see dispatch_workspace_size); the only process-wide setting
 *     is the guard on in-kernel waits (dispatch_set_wait_limit).
 *   - Language: the header is plain C (C99) as well as C++. A compiler other
 *     than hipcc must define __HIP_PLATFORM_AMD__, as HIP's own runtime header
 *     included below requires.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DISPATCH_ABI_VERSION 6

/* Limits. K <= 32 follows the page's bound on the top-k width (section 4.2);
 * R <= 1024 follows its kNumMaxRanks (section 6.2). */
#define DISPATCH_MAX_TOPK 32
#define DISPATCH_MAX_EXPERTS 4096
#define DISPATCH_MAX_RANKS 1024

/* Host error codes (returned before any work is enqueued). */
#define DISPATCH_OK 0
#define DISPATCH_ERR_NULL (-1)      /* a required pointer is NULL */
#define DISPATCH_ERR_ARG (-2)       /* a size or flag is out of range */
#define DISPATCH_ERR_ALIGN (-3)     /* row_bytes % 16 != 0 or a pointer is misaligned */
#define DISPATCH_ERR_WORKSPACE (-4) /* workspace missing, too small or misaligned */
#define DISPATCH_ERR_HIP (-5)       /* the HIP runtime refused a launch */

/* Device status bits written by dispatch_layout to *status. */
#define DISPATCH_STATUS_BAD_EXPERT 1u     /* an entry of topk_idx is >= num_experts */
#define DISPATCH_STATUS_RECV_OVERFLOW 2u  /* expert_psum[E] > recv_capacity_rows */
#define DISPATCH_STATUS_RANK_OVERFLOW 4u  /* rank_psum[R] > rank_capacity_rows */
#define DISPATCH_STATUS_DUP_EXPERT 8u     /* an expert repeated within one token */
#define DISPATCH_STATUS_BAD_COUNT 16u     /* expand: a recv_count outside [0, rows_per_source] */
#define DISPATCH_STATUS_TIMEOUT 32u       /* one-launch layout: a tile's bounded wait for the other
                                             tiles ran out (a guard, see dispatch_set_wait_limit);
                                             slot maps, inverse maps and rows are unspecified */

/* Output selection for dispatch_scatter. */
#define DISPATCH_RANK_CONTIG 1u  /* write rank_x (and rank_sf) */
#define DISPATCH_EXPERT_MAJOR 2u /* write recv_x (and recv_sf) */
#define DISPATCH_ZERO_PAD 4u     /* zero the alignment pad rows of recv_x / recv_sf */
#define DISPATCH_ALL_OUTPUTS (DISPATCH_RANK_CONTIG | DISPATCH_EXPERT_MAJOR | DISPATCH_ZERO_PAD)
/* A hint for dispatch_scatter, changing no result: the token rows were just
 * read into the Infinity Cache (by dispatch_layout_read_ahead, on the same
 * stream). The scatter then keeps fewer row stores in flight per CU, which on
 * MI355X moves rows from the cache faster (and rows from HBM slower). It is
 * ignored where dispatch_layout_read_ahead reads nothing (rows and scale
 * factors above 160 MB) and by the layout calls; dispatch_layout_and_scatter
 * sets it itself when it reads the rows ahead. */
#define DISPATCH_ROWS_READ_AHEAD 8u

typedef struct dispatch_problem {
    int64_t num_tokens;         /* T >= 0 */
    int32_t num_topk;           /* K, 1..DISPATCH_MAX_TOPK */
    int32_t num_experts;        /* E, 1..DISPATCH_MAX_EXPERTS */
    int32_t num_ranks;          /* R, 1..DISPATCH_MAX_RANKS, E % R == 0 */
    int32_t expert_alignment;   /* A >= 1; 1 = no padding (section 7.2) */
    int32_t topk_idx_bytes;     /* width of a topk_idx entry: 8 (int64) or 4 (int32) */
    int32_t sf_per_token;       /* S >= 0 fp32 scale factors per token (H/128 for fp8, else 0) */
    int64_t row_bytes;          /* bytes per token row (H * element size), multiple of 16, 16..2^31-16 */
    int64_t recv_capacity_rows; /* rows of recv_x / recv_sf / recv_src_token_idx */
    int64_t rank_capacity_rows; /* rows of rank_x / rank_sf / rank_src_token_idx */
    uint32_t flags;             /* DISPATCH_* output selection and DISPATCH_ROWS_READ_AHEAD, used by dispatch_scatter */
    uint32_t reserved;          /* must be 0 */
} dispatch_problem_t;

/* Layout outputs; every pointer is a caller-owned device int32 array. */
typedef struct dispatch_layout {
    int32_t* expert_count;       /* [E]   routed pairs per expert, before alignment */
    int32_t* rank_count;         /* [R]   tokens per rank, deduplicated (section 4.2) */
    int32_t* expert_psum;        /* [E+1] exclusive psum of align(expert_count, A); [E] = total rows */
    int32_t* rank_psum;          /* [R+1] exclusive psum of rank_count; [R] = total rank rows */
    int32_t* expert_slot;        /* [T*K] recv_x row of pair (t, k), -1 if masked */
    int32_t* rank_slot;          /* [T*K] rank_x row of (t, rank of k) at the owning k, else -1 */
    int32_t* recv_src_token_idx; /* [recv_capacity_rows] token of each recv_x row, -1 on pads */
    int32_t* rank_src_token_idx; /* [rank_capacity_rows] token of each rank_x row */
    int32_t* status;             /* [1]   DISPATCH_STATUS_* bits, 0 = success */
    /* Optional (NULL = off), caller-owned and kept across calls: [E] running
     * totals of expert_count. A call that ends with status 0 adds its
     * expert_count to it with device atomics, so calls on several streams may
     * share one array; a failed call adds nothing. The page's cumulative
     * per-expert receive statistics (section 7.2), an int32 counter there too:
     * it wraps modulo 2^32, so a caller that keeps it over more than 2^31 rows
     * per expert reads and clears it from time to time. */
    int32_t* expert_count_cumulative;
} dispatch_layout_t;

/* Version of this ABI (DISPATCH_ABI_VERSION). */
int dispatch_abi_version(void);

/* Static, human-readable text for a host error code. Never NULL. */
const char* dispatch_strerror(int code);

/* Bytes of device workspace the dispatch layout calls need for this problem
 * (T, K, E, R are read). The workspace must be 256-byte aligned and
 * zero-filled before its first use (hipMemset to 0 once). It holds per-tile
 * histograms, which each call rewrites before reading, and the words through
 * which the tiles of a one-launch layout exchange their key counts (section
 * 4.5's cross-tile merge): every call leaves those zero again when it ends,
 * so a workspace stays ready for the next call of any problem that fits it,
 * dispatch or expand. Nothing else may write into it. */
int dispatch_workspace_size(const dispatch_problem_t* problem, size_t* bytes);

/* Worst-case row counts, for sizing outputs without reading the totals back:
 * max_recv_rows = T*K + E*(A-1) and max_rank_rows = T*min(K, R). Either
 * output pointer may be NULL. */
int dispatch_max_rows(const dispatch_problem_t* problem, int64_t* max_recv_rows,
                      int64_t* max_rank_rows);

/* Count -> Prefix Sum -> slot assignment (sections 4, 5, 6.2, 6.4 and 7).
 * topk_idx: device [T, K] row-major of problem->topk_idx_bytes wide signed
 * integers; a negative entry is masked. Writes every field of `out` (counts
 * and psums always; slot and inverse maps when *status is 0). Needs
 * `workspace` of at least dispatch_workspace_size() bytes. A batch of one
 * tile takes one kernel, larger batches a count kernel and an assign kernel,
 * or three kernels with a column scan (dispatch_kernel_count tells which). */
int dispatch_layout(const dispatch_problem_t* problem, const void* topk_idx,
                    const dispatch_layout_t* out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* dispatch_layout, and while it runs, a read of the token rows x
 * [T, row_bytes] (16-byte aligned) and of x_sf [T, S] (may be NULL) that
 * leaves them in the GPU's Infinity Cache for a dispatch_scatter of the same
 * rows that follows. The layout kernels are latency-bound and leave HBM
 * idle; the scatter reads every live row once while it writes about
 * fourteen times as many bytes, and rows it finds in the cache no longer
 * interleave HBM reads into that write stream. Rows and scale factors of
 * more than 160 MB together are not read (they would push their own first
 * rows out of the 256 MB cache). The scatter that follows is told so by
 * DISPATCH_ROWS_READ_AHEAD in its problem's flags. Rows that are read ahead
 * let a batch of up to 256 tiles be laid out in one launch: each tile's
 * workgroup ranks its pairs once, hands its key counts to the others
 * through the workspace, waits for theirs (all tiles are resident together;
 * the wait is bounded, see dispatch_set_wait_limit) and assigns its slots,
 * while the launch's other workgroups read the rows. Outputs, checks and
 * errors are those of
 * dispatch_layout, plus DISPATCH_ERR_ALIGN for a misaligned x or x_sf;
 * nothing beyond the layout outputs is written. (Not a step of the page's
 * method: a measure for MI355X's memory hierarchy.) */
int dispatch_layout_read_ahead(const dispatch_problem_t* problem, const void* topk_idx,
                               const dispatch_layout_t* out, void* workspace, size_t workspace_bytes,
                               const void* x, const float* x_sf, hipStream_t stream);

/* Row scatter of a layout made by dispatch_layout with the same problem
 * (sections 6.3, 7.3 and 8.2). Reads layout->expert_count, expert_psum,
 * expert_slot, rank_slot and status. x: device [T, row_bytes] (opaque bytes,
 * bf16 or fp8 alike), 16-byte aligned. x_sf: device fp32 [T, S] or NULL when
 * S == 0. Writes, as selected by problem->flags:
 *   rank_x [rank_psum[R], row_bytes] and rank_sf [rank_psum[R], S];
 *   recv_x [expert_psum[E], row_bytes] and recv_sf [expert_psum[E], S], with
 *   pad rows zeroed under DISPATCH_ZERO_PAD.
 * Copies are bitwise. Writes nothing when the layout's status is non-zero.
 * One wavefront copies each 1 KB of a row (4 KB when rows have about one
 * destination; after a read-ahead, one workgroup of ceil((K + min(K, R)) / 4)
 * wavefronts per 1 KB), and the launch must fit one grid: at most 2^31 - 1
 * workgroups and 2^32 - 1 work-items. A larger problem returns
 * DISPATCH_ERR_ARG before anything is enqueued.
 * A layout may be kept and scattered again, for new rows of the same routing,
 * without recomputing it (the page's cached dispatch, section 6.2). */
int dispatch_scatter(const dispatch_problem_t* problem, const dispatch_layout_t* layout,
                     const void* x, const float* x_sf, void* rank_x, float* rank_sf,
                     void* recv_x, float* recv_sf, hipStream_t stream);

/* dispatch_layout followed by dispatch_scatter in one call, with the same
 * arguments, checks, outputs and status semantics as those two calls made in
 * turn (the layout reads the rows ahead, as dispatch_layout_read_ahead, and
 * the scatter then runs as with DISPATCH_ROWS_READ_AHEAD). A small batch
 * (T * K up to 3072 pairs, or 2048 when pad rows are
 * zeroed; fewer when E + R is large) is laid out and copied by a single
 * kernel: every workgroup ranks the whole batch itself, so none waits for
 * another, and each copies its share of the rows' 1 KB segments. That saves
 * one or two launches, the dominant cost of small (decode-sized) batches.
 * Larger batches run the layout kernel(s) and the scatter kernel. */
int dispatch_layout_and_scatter(const dispatch_problem_t* problem, const void* topk_idx,
                                const dispatch_layout_t* out, void* workspace, size_t workspace_bytes,
                                const void* x, const float* x_sf, void* rank_x, float* rank_sf,
                                void* recv_x, float* recv_sf, hipStream_t stream);

/* dispatch_layout_and_scatter without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The layout's workspace is a
 * device array of DISPATCH_NOALLOC_WORKSPACE_BYTES inside the library (one
 * per GPU, held until the process ends); the call allocates nothing. A
 * problem whose dispatch_workspace_size() exceeds that size returns
 * DISPATCH_ERR_WORKSPACE before anything is enqueued; every other argument,
 * check and output is that of dispatch_layout_and_scatter. The array starts
 * zeroed and every call leaves it ready for the next, but calls that overlap
 * in time on one GPU (concurrent streams) share it and race: serialize them,
 * or use dispatch_layout_and_scatter with a workspace per stream. */
#define DISPATCH_NOALLOC_WORKSPACE_BYTES 4194304 /* 4 MiB */
int dispatch_layout_and_scatter_noalloc(const dispatch_problem_t* problem, const void* topk_idx,
                                        const dispatch_layout_t* out, const void* x, const float* x_sf,
                                        void* rank_x, float* rank_sf, void* recv_x, float* recv_sf,
                                        hipStream_t stream);

/* Kernels the calls above launch for this problem (its T, K, E, R,
 * row_bytes and S are read): *layout_kernels for dispatch_layout (1 when one
 * tile holds the batch, 2 with the tile histograms reduced in an assign
 * kernel, 3 with the column scan) and *layout_and_scatter_kernels for
 * dispatch_layout_and_scatter (1 on its one-kernel path; 2 when its layout,
 * reading the rows ahead, is one launch; else the layout's kernels plus the
 * scatter). Either pointer may be NULL. */
int dispatch_kernel_count(const dispatch_problem_t* problem, int* layout_kernels,
                          int* layout_and_scatter_kernels);

/* Bound on the in-kernel wait of the one-launch layout (the layout of
 * dispatch_layout_read_ahead and dispatch_layout_and_scatter), in polls of the
 * other tiles' words (about a microsecond each). The tiles are the first
 * workgroups of their launch and wait only for each other, so the wait ends
 * without it; the bound is a guard, after which a tile writes nothing and the
 * call reports DISPATCH_STATUS_TIMEOUT (its workspace stays ready for the
 * next call). polls = 0 restores the default of 2^20; a small bound forces
 * the timeout path, for tests. A process-wide setting read when a call is
 * enqueued; returns DISPATCH_ERR_ARG for a negative bound. */
#define DISPATCH_DEFAULT_WAIT_LIMIT 1048576
int dispatch_set_wait_limit(int64_t polls);

/* ---------------------------------------------------------------------------
 * Receiver-side expand (the page's copy epilogue: sections 3, 6.4, 8.2, 8.3
 * and 12). A receiver rank holds the rows S source ranks sent it in a receive
 * buffer with a fixed stride of rows_per_source rows per source (the page's
 * kNumMaxTokensPerRank); source s sent recv_count[s] rows, the first ones of
 * its region, and every row comes with its token's K global expert ids. The
 * receiver owns the experts [local_rank*E/R, (local_rank+1)*E/R) and builds
 * the expert-major layout over them: rows of a local expert follow (source,
 * row) order, buckets are padded to the expert alignment.
 * ------------------------------------------------------------------------- */
typedef struct dispatch_expand_problem {
    int32_t num_sources;        /* S >= 1 */
    int32_t rows_per_source;    /* M >= 0 rows of the receive buffer per source */
    int32_t num_topk;           /* K, 1..DISPATCH_MAX_TOPK */
    int32_t num_experts;        /* E of the sending side (global ids), 1..DISPATCH_MAX_EXPERTS */
    int32_t num_ranks;          /* R, 1..DISPATCH_MAX_RANKS, E % R == 0 */
    int32_t local_rank;         /* this receiver, 0..R-1 */
    int32_t expert_alignment;   /* A >= 1 */
    int32_t topk_idx_bytes;     /* 8 (int64) or 4 (int32) */
    int32_t sf_per_token;       /* fp32 scale factors per row, >= 0 */
    uint32_t reserved;          /* must be 0 */
    int64_t row_bytes;          /* bytes per row, multiple of 16, 16..2^31-16 (expand_scatter only) */
    int64_t recv_capacity_rows; /* rows of the expert-major output */
} dispatch_expand_problem_t;

/* Workspace bytes for dispatch_expand_layout (same layout and rules as the
 * dispatch's: 256-byte aligned, zero-filled before its first use, so that
 * one buffer may serve calls of either kind; the expand's own kernels never
 * write its exchange region). */
int dispatch_expand_workspace_size(const dispatch_expand_problem_t* problem, size_t* bytes);

/* Worst-case expert-major rows: S*M*min(K, E/R) + (E/R)*(A-1). */
int dispatch_expand_max_rows(const dispatch_expand_problem_t* problem, int64_t* max_recv_rows);

/* Expert-major layout of a receive buffer. recv_topk_idx: device [S*M, K]
 * global expert ids (rows past a source's count are never read). recv_count:
 * device int32 [S]. `out` uses dispatch_layout_t with its rank fields NULL:
 * expert_count[E/R], expert_psum[E/R+1], expert_slot[S*M*K] (-1 for another
 * rank's expert, a masked entry or an unused row), recv_src_token_idx
 * [recv_capacity_rows] holding the receive-buffer row of each slot (-1 on
 * pads), the optional expert_count_cumulative[E/R] (the local experts' rows
 * received over all calls), status (DISPATCH_STATUS_*; BAD_EXPERT for an id >= E, DUP_EXPERT for
 * a local expert twice in a row, BAD_COUNT for a count outside [0, M]). */
int dispatch_expand_layout(const dispatch_expand_problem_t* problem, const void* recv_topk_idx,
                           const int32_t* recv_count, const dispatch_layout_t* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* dispatch_expand_layout followed by dispatch_expand_scatter in one call, with
 * the same arguments, checks and outputs as those two calls made in turn. A
 * small receive buffer (S * M * K up to 2048 entries) is laid out and copied
 * by one kernel, as in dispatch_layout_and_scatter. */
int dispatch_expand_layout_and_scatter(const dispatch_expand_problem_t* problem, const void* recv_topk_idx,
                                       const int32_t* recv_count, const dispatch_layout_t* out, void* workspace,
                                       size_t workspace_bytes, const void* recv_buf, const float* recv_sf_buf,
                                       void* recv_x, float* recv_sf, hipStream_t stream);

/* Copies the received rows (recv_buf [S*M, row_bytes], recv_sf_buf [S*M, sf])
 * into the expert-major recv_x / recv_sf of a layout made by
 * dispatch_expand_layout, zeroing pad rows. Writes nothing when the layout's
 * status is non-zero. */
int dispatch_expand_scatter(const dispatch_expand_problem_t* problem, const dispatch_layout_t* layout,
                            const void* recv_buf, const float* recv_sf_buf, void* recv_x, float* recv_sf,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Combine: the reverse of the expert-major scatter, reusing the layout's slot
 * map (the page keeps it for the combine kernel, section 6.2):
 *   out[t, :] = sum over k with expert_slot[t, k] >= 0 of
 *               topk_weights[t, k] * y[expert_slot[t, k], :]
 * y and out are bf16; the sum is taken in fp32 with one fused multiply-add
 * per routed k in ascending k order from 0, then rounded to bf16 to nearest,
 * ties to even. A token with no routed entry gets a zero row.
 * ------------------------------------------------------------------------- */
typedef struct dispatch_combine_problem {
    int64_t num_tokens;   /* T >= 0 */
    int32_t num_topk;     /* K, 1..DISPATCH_MAX_TOPK */
    uint32_t reserved;    /* must be 0 */
    int64_t hidden;       /* H: bf16 elements per row, multiple of 8, 8..2^30-8 */
    int64_t expert_rows;  /* rows of y; every slot must be below it (others are dropped) */
} dispatch_combine_problem_t;

/* expert_slot: device int32 [T, K] (from dispatch_layout); topk_weights:
 * device fp32 [T, K]; y: device bf16 [expert_rows, H], 16-byte aligned;
 * out: device bf16 [T, H], 16-byte aligned. */
int dispatch_combine(const dispatch_combine_problem_t* problem, const int32_t* expert_slot,
                     const float* topk_weights, const void* y, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H */
