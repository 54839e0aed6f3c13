/*
 * CPU oracle for MoE dispatch layout and scatter: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, single-threaded, deliberately slow C implementation of what the
 * dispatch counting sort computes ("DeepEP Counting Sort / Bucketization" page:
 * Count -> Prefix Sum -> Scatter, sections 4 to 8). Only the tests, the smoke
 * check and the benchmark's CPU baseline call it; the product path never does.
 * It shares no code, header or table with the HIP library.
 *
 * Conventions (the readings taken where the page is silent are listed in the
 * repository's design notes):
 *   - topk_idx[T, K] is int64; any negative entry is a masked pair.
 *   - A "rank" is a group of E/R consecutive experts: r = e / (E/R).
 *   - expert_psum[E+1] and rank_psum[R+1] are exclusive prefix sums; the
 *     expert psum runs over counts aligned up to a multiple of A.
 *   - Slots inside an expert bucket or a rank block follow ascending token index.
 *   - The (token, rank) slot is held by the highest k of that rank in the token;
 *     the other k of the same rank get -1.
 *
 * Status bits returned (same meaning as the device status word):
 *   1 = expert id >= E, 2 = expert-major rows exceed capacity,
 *   4 = rank rows exceed capacity, 8 = an expert repeated within one token.
 */
#ifndef MOE_DISPATCH_ORACLE_H
#define MOE_DISPATCH_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_BAD_EXPERT 1
#define ORACLE_RECV_OVERFLOW 2
#define ORACLE_RANK_OVERFLOW 4
#define ORACLE_DUP_EXPERT 8
#define ORACLE_BAD_ARGS (-1)

/* Counts, prefix sums and slot maps. Outputs are caller-owned host arrays:
 * expert_count[E], rank_count[R], expert_psum[E+1], rank_psum[R+1],
 * expert_slot[T*K], rank_slot[T*K], recv_src_token_idx[recv_capacity],
 * rank_src_token_idx[rank_capacity]. Counts and psums are always written;
 * slots and inverse maps only when the returned status is 0. */
int oracle_dispatch_layout(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                           int32_t num_ranks, int32_t expert_alignment,
                           const int64_t* topk_idx, int64_t recv_capacity,
                           int64_t rank_capacity, int32_t* expert_count,
                           int32_t* rank_count, int32_t* expert_psum, int32_t* rank_psum,
                           int32_t* expert_slot, int32_t* rank_slot,
                           int32_t* recv_src_token_idx, int32_t* rank_src_token_idx);

/* Row copies driven by a layout: rank_x[rank_slot] = x[t] once per (token, rank),
 * recv_x[expert_slot] = x[t] per valid pair, scale-factor rows alike, and the
 * alignment pad rows of recv_x / recv_sf set to zero bytes. Scale factors are
 * moved as raw 32-bit words. Any of the output pointers may be NULL to skip
 * that output. */
int oracle_dispatch_scatter(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                            int64_t row_bytes, int32_t sf_per_token, const uint8_t* x,
                            const uint32_t* x_sf, const int32_t* expert_count,
                            const int32_t* expert_psum, const int32_t* expert_slot,
                            const int32_t* rank_slot, uint8_t* rank_x, uint32_t* rank_sf,
                            uint8_t* recv_x, uint32_t* recv_sf, int zero_pad);

/* Receiver side of the expand (the page's copy epilogue: sections 3, 6.4
 * and 8.2-8.3): rows received from S source ranks sit in a receive buffer
 * with M rows per source; source s sent recv_count[s] rows, each carrying its
 * token's top-k global expert ids recv_topk[S*M, K]. This receiver owns the
 * experts [local_rank*E/R, (local_rank+1)*E/R). Outputs, over those local
 * experts: expert_count[E/R], expert_psum[E/R+1] (aligned, exclusive),
 * expert_slot[S*M*K] (-1 for non-local or unused entries) and
 * recv_src_row_idx[recv_capacity] (received row index of each slot, -1 on
 * pads). Rows inside a local expert's bucket follow (source, row) order.
 * Status: 1 = expert id >= E, 2 = rows exceed capacity, 8 = a local expert
 * repeated within a row, 16 = a recv_count outside [0, M]. */
#define ORACLE_BAD_COUNT 16
int oracle_expand_layout(int32_t num_sources, int32_t rows_per_source, int32_t num_topk,
                         int32_t num_experts, int32_t num_ranks, int32_t local_rank,
                         int32_t expert_alignment, const int64_t* recv_topk,
                         const int32_t* recv_count, int64_t recv_capacity,
                         int32_t* expert_count, int32_t* expert_psum, int32_t* expert_slot,
                         int32_t* recv_src_row_idx);

/* Combine, the reverse of the expert-major scatter: out[t, h] = sum over the
 * token's routed k of weight[t, k] * y[expert_slot[t, k], h]. y is bf16
 * [rows, H] (raw 16-bit patterns), weights fp32 [T, K]; the sum is taken in
 * double precision (exact up to double rounding) and written as double
 * [T, H]. Entries with expert_slot < 0 contribute nothing. Returns -1 for a
 * slot >= rows. */
int oracle_combine(int64_t num_tokens, int32_t num_topk, int64_t hidden, int64_t rows,
                   const uint16_t* y, const float* weights, const int32_t* expert_slot, double* out);

#ifdef __cplusplus
}
#endif

#endif
