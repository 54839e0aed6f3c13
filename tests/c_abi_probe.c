/* Built as C99 by tests/test_c_header.py: the public header must compile as
 * plain C, and the struct layouts and host-only results it gives a C caller
 * must be the ones the Python binding uses. Prints one "key value" per line. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "moe_dispatch.h"

#define SIZE(T) printf("sizeof.%s %zu\n", #T, sizeof(T))
#define OFF(T, f) printf("offset.%s.%s %zu\n", #T, #f, offsetof(T, f))

int main(void) {
    printf("abi %d\n", dispatch_abi_version());
    printf("macro_abi %d\n", DISPATCH_ABI_VERSION);

    SIZE(dispatch_problem_t);
    OFF(dispatch_problem_t, num_tokens);
    OFF(dispatch_problem_t, num_topk);
    OFF(dispatch_problem_t, num_experts);
    OFF(dispatch_problem_t, num_ranks);
    OFF(dispatch_problem_t, expert_alignment);
    OFF(dispatch_problem_t, topk_idx_bytes);
    OFF(dispatch_problem_t, sf_per_token);
    OFF(dispatch_problem_t, row_bytes);
    OFF(dispatch_problem_t, recv_capacity_rows);
    OFF(dispatch_problem_t, rank_capacity_rows);
    OFF(dispatch_problem_t, flags);
    OFF(dispatch_problem_t, reserved);

    SIZE(dispatch_layout_t);
    OFF(dispatch_layout_t, expert_count);
    OFF(dispatch_layout_t, rank_count);
    OFF(dispatch_layout_t, expert_psum);
    OFF(dispatch_layout_t, rank_psum);
    OFF(dispatch_layout_t, expert_slot);
    OFF(dispatch_layout_t, rank_slot);
    OFF(dispatch_layout_t, recv_src_token_idx);
    OFF(dispatch_layout_t, rank_src_token_idx);
    OFF(dispatch_layout_t, status);
    OFF(dispatch_layout_t, expert_count_cumulative);

    SIZE(dispatch_expand_problem_t);
    OFF(dispatch_expand_problem_t, num_sources);
    OFF(dispatch_expand_problem_t, rows_per_source);
    OFF(dispatch_expand_problem_t, num_topk);
    OFF(dispatch_expand_problem_t, num_experts);
    OFF(dispatch_expand_problem_t, num_ranks);
    OFF(dispatch_expand_problem_t, local_rank);
    OFF(dispatch_expand_problem_t, expert_alignment);
    OFF(dispatch_expand_problem_t, topk_idx_bytes);
    OFF(dispatch_expand_problem_t, sf_per_token);
    OFF(dispatch_expand_problem_t, reserved);
    OFF(dispatch_expand_problem_t, row_bytes);
    OFF(dispatch_expand_problem_t, recv_capacity_rows);

    SIZE(dispatch_combine_problem_t);
    OFF(dispatch_combine_problem_t, num_tokens);
    OFF(dispatch_combine_problem_t, num_topk);
    OFF(dispatch_combine_problem_t, reserved);
    OFF(dispatch_combine_problem_t, hidden);
    OFF(dispatch_combine_problem_t, expert_rows);

    /* Host-only calls on the 4096-token, 7168-wide bf16 batch, top-8 of 256
     * experts in 8 ranks, alignment 1, and on the same batch at alignment 128. */
    for (int a = 1; a <= 128; a += 127) {
        dispatch_problem_t p = {0};
        p.num_tokens = 4096;
        p.num_topk = 8;
        p.num_experts = 256;
        p.num_ranks = 8;
        p.expert_alignment = a;
        p.topk_idx_bytes = 8;
        p.row_bytes = 14336;
        p.flags = DISPATCH_ALL_OUTPUTS;
        int64_t max_recv = 0, max_rank = 0;
        int rc = dispatch_max_rows(&p, &max_recv, &max_rank);
        printf("max_rows.a%d %d %lld %lld\n", a, rc, (long long)max_recv, (long long)max_rank);
        p.recv_capacity_rows = max_recv;
        p.rank_capacity_rows = max_rank;
        size_t ws = 0;
        rc = dispatch_workspace_size(&p, &ws);
        printf("workspace.a%d %d %zu\n", a, rc, ws);
        int lk = 0, bk = 0;
        rc = dispatch_kernel_count(&p, &lk, &bk);
        printf("kernels.a%d %d %d %d\n", a, rc, lk, bk);
    }
    /* A host error: E not a multiple of R. */
    dispatch_problem_t bad = {0};
    bad.num_tokens = 1;
    bad.num_topk = 1;
    bad.num_experts = 10;
    bad.num_ranks = 4;
    bad.expert_alignment = 1;
    bad.topk_idx_bytes = 8;
    bad.row_bytes = 16;
    size_t ws_bad = 0;
    printf("bad_workspace %d\n", dispatch_workspace_size(&bad, &ws_bad));
    printf("strerror_arg %s\n", dispatch_strerror(DISPATCH_ERR_ARG));
    return 0;
}
