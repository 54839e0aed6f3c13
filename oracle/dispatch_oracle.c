/*
 * CPU oracle for MoE dispatch layout and scatter: TEST INFRASTRUCTURE ONLY.
 *
 * Plain single-threaded C, written for a reader to check by eye against the
 * "DeepEP Counting Sort / Bucketization" page. It takes the page's steps in the
 * page's order: Count (section 4.2), Prefix Sum with expert alignment
 * (sections 5.2 and 7.2), the rank-level and expert-level slot scatters
 * (sections 6.2 and 6.4) and the row copies with zero padding (sections 6.3,
 * 7.3 and 8.2). Where the page's kernel lets atomics decide the order inside a
 * bucket, this oracle fixes ascending token order, which makes the result
 * unique. Two further steps follow the same page: the receiver-side expand
 * of a fixed-stride receive buffer (its copy epilogue, sections 3, 6.4 and
 * 8.2-8.3), in (source, row) order, and the combine that the page's slot map
 * is kept for (section 6.2), summed in double precision. Only tests, the
 * smoke check and the benchmark's CPU baseline may call it; the product path
 * never links or loads it.
 */
#include "dispatch_oracle.h"

#include <stdlib.h>
#include <string.h>

/* The value of a bfloat16 bit pattern: the upper half of an IEEE binary32. */
static double bf16_value(uint16_t bits) {
    const uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* ceil(c / a) * a, the page's math::align (section 7.2); align(0, a) = 0 and
 * an alignment of 1 leaves the count unchanged. */
static int64_t align_up(int64_t c, int64_t a) {
    if (a <= 1) return c;
    return ((c + a - 1) / a) * a;
}

/* True when entry (t, k) names an expert that exists (masked entries are
 * negative; the page's code keeps only ids >= 0, section 4.2). */
static int is_routed(int64_t e, int32_t num_experts) { return e >= 0 && e < num_experts; }

int oracle_dispatch_layout(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                           int32_t num_ranks, int32_t expert_alignment,
                           const int64_t* topk_idx, int64_t recv_capacity,
                           int64_t rank_capacity, int32_t* expert_count,
                           int32_t* rank_count, int32_t* expert_psum, int32_t* rank_psum,
                           int32_t* expert_slot, int32_t* rank_slot,
                           int32_t* recv_src_token_idx, int32_t* rank_src_token_idx) {
    const int64_t T = num_tokens;
    const int32_t K = num_topk, E = num_experts, R = num_ranks, A = expert_alignment;
    if (T < 0 || K < 1 || K > 32 || E < 1 || R < 1 || E % R != 0 || A < 1) return ORACLE_BAD_ARGS;
    if (T * K + (int64_t)E * (A - 1) > INT32_MAX) return ORACLE_BAD_ARGS;
    const int32_t experts_per_rank = E / R;
    int status = 0;

    /* ---- Count (section 4.2). Every routed pair adds one to its expert. A
     * token adds one to a rank however many of its experts live there: only
     * the highest k of that rank in the token (the page's "master lane" of
     * the deduplicate step) counts it. Expert ids >= E are reported and
     * skipped; a repeated expert within a token breaks the page's stated
     * precondition and is reported too. */
    for (int32_t e = 0; e < E; ++e) expert_count[e] = 0;
    for (int32_t r = 0; r < R; ++r) rank_count[r] = 0;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t* row = topk_idx + t * K;
        for (int32_t k = 0; k < K; ++k) {
            const int64_t e = row[k];
            if (e < 0) continue;
            if (e >= E) {
                status |= ORACLE_BAD_EXPERT;
                continue;
            }
            for (int32_t j = 0; j < k; ++j)
                if (row[j] == e) status |= ORACLE_DUP_EXPERT;
            expert_count[e] += 1;
            const int64_t r = e / experts_per_rank;
            int owner = 1;
            for (int32_t j = k + 1; j < K; ++j)
                if (is_routed(row[j], E) && row[j] / experts_per_rank == r) owner = 0;
            if (owner) rank_count[r] += 1;
        }
    }

    /* ---- Prefix sum (sections 5.2 and 7.2). Exclusive, n+1 outputs; the
     * expert counts are aligned up before they are summed, the rank counts
     * are summed as they are. */
    int64_t run = 0;
    expert_psum[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        run += align_up(expert_count[e], A);
        expert_psum[e + 1] = (int32_t)run;
    }
    run = 0;
    rank_psum[0] = 0;
    for (int32_t r = 0; r < R; ++r) {
        run += rank_count[r];
        rank_psum[r + 1] = (int32_t)run;
    }
    if (expert_psum[E] > recv_capacity) status |= ORACLE_RECV_OVERFLOW;
    if (rank_psum[R] > rank_capacity) status |= ORACLE_RANK_OVERFLOW;
    if (status) return status;

    /* ---- Slot scatter (sections 6.2 and 6.4). A cursor per expert and per
     * rank starts at the exclusive prefix sum; walking tokens in ascending
     * order, each pair takes its expert cursor and each (token, rank) takes
     * its rank cursor at the owning k. Slots between an expert's last pair and
     * the next expert's start are alignment pads and map back to token -1. */
    int64_t* expert_cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
    int64_t* rank_cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)R);
    if (!expert_cursor || !rank_cursor) {
        free(expert_cursor);
        free(rank_cursor);
        return ORACLE_BAD_ARGS;
    }
    for (int32_t e = 0; e < E; ++e) expert_cursor[e] = expert_psum[e];
    for (int32_t r = 0; r < R; ++r) rank_cursor[r] = rank_psum[r];
    for (int64_t s = 0; s < expert_psum[E]; ++s) recv_src_token_idx[s] = -1;

    for (int64_t t = 0; t < T; ++t) {
        const int64_t* row = topk_idx + t * K;
        for (int32_t k = 0; k < K; ++k) {
            const int64_t e = row[k];
            if (e < 0) {
                expert_slot[t * K + k] = -1;
                rank_slot[t * K + k] = -1;
                continue;
            }
            const int64_t slot = expert_cursor[e]++;
            expert_slot[t * K + k] = (int32_t)slot;
            recv_src_token_idx[slot] = (int32_t)t;

            const int64_t r = e / experts_per_rank;
            int owner = 1;
            for (int32_t j = k + 1; j < K; ++j)
                if (is_routed(row[j], E) && row[j] / experts_per_rank == r) owner = 0;
            if (owner) {
                const int64_t rank_row = rank_cursor[r]++;
                rank_slot[t * K + k] = (int32_t)rank_row;
                rank_src_token_idx[rank_row] = (int32_t)t;
            } else {
                rank_slot[t * K + k] = -1;
            }
        }
    }
    free(expert_cursor);
    free(rank_cursor);
    return 0;
}

int oracle_dispatch_scatter(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                            int64_t row_bytes, int32_t sf_per_token, const uint8_t* x,
                            const uint32_t* x_sf, const int32_t* expert_count,
                            const int32_t* expert_psum, const int32_t* expert_slot,
                            const int32_t* rank_slot, uint8_t* rank_x, uint32_t* rank_sf,
                            uint8_t* recv_x, uint32_t* recv_sf, int zero_pad) {
    const int64_t T = num_tokens;
    const int32_t K = num_topk, S = sf_per_token;
    if (T < 0 || K < 1 || row_bytes < 0 || S < 0) return ORACLE_BAD_ARGS;
    const size_t sf_bytes = sizeof(uint32_t) * (size_t)S;

    /* Rank-level scatter (sections 6.2 and 6.3): one copy of the token's row
     * per destination rank, at the slot its owning k holds. */
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            const int64_t row = rank_slot[t * K + k];
            if (row < 0) continue;
            if (rank_x) memcpy(rank_x + row * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            if (rank_sf && S) memcpy(rank_sf + row * S, x_sf + t * S, sf_bytes);
        }
    }
    /* Expert-level scatter (sections 6.4 and 8.2): one copy per routed pair
     * into the expert-major buffer. */
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            const int64_t slot = expert_slot[t * K + k];
            if (slot < 0) continue;
            if (recv_x) memcpy(recv_x + slot * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            if (recv_sf && S) memcpy(recv_sf + slot * S, x_sf + t * S, sf_bytes);
        }
    }
    /* Zero padding (section 7.3): the slots after each expert's real rows up
     * to its aligned end hold zero bytes. */
    if (zero_pad) {
        for (int32_t e = 0; e < num_experts; ++e) {
            for (int64_t s = (int64_t)expert_psum[e] + expert_count[e]; s < expert_psum[e + 1]; ++s) {
                if (recv_x) memset(recv_x + s * row_bytes, 0, (size_t)row_bytes);
                if (recv_sf && S) memset(recv_sf + s * S, 0, sf_bytes);
            }
        }
    }
    return 0;
}

int oracle_expand_layout(int32_t num_sources, int32_t rows_per_source, int32_t num_topk,
                         int32_t num_experts, int32_t num_ranks, int32_t local_rank,
                         int32_t expert_alignment, const int64_t* recv_topk,
                         const int32_t* recv_count, int64_t recv_capacity,
                         int32_t* expert_count, int32_t* expert_psum, int32_t* expert_slot,
                         int32_t* recv_src_row_idx) {
    const int32_t S = num_sources, M = rows_per_source, K = num_topk, E = num_experts, R = num_ranks;
    const int32_t A = expert_alignment;
    if (S < 1 || M < 0 || K < 1 || K > 32 || E < 1 || R < 1 || E % R != 0 || local_rank < 0 ||
        local_rank >= R || A < 1)
        return ORACLE_BAD_ARGS;
    const int32_t L = E / R;                  /* local experts */
    const int64_t first_expert = (int64_t)local_rank * L;
    const int64_t rows = (int64_t)S * M;
    if (rows * K + (int64_t)L * (A - 1) > INT32_MAX) return ORACLE_BAD_ARGS;
    int status = 0;

    /* Received rows: the first recv_count[s] rows of source s's region; the
     * rest of the region was never written by that source. */
    for (int32_t s = 0; s < S; ++s)
        if (recv_count[s] < 0 || recv_count[s] > M) status |= ORACLE_BAD_COUNT;

    /* Count the pairs of every local expert over the received rows. */
    for (int32_t e = 0; e < L; ++e) expert_count[e] = 0;
    for (int32_t s = 0; s < S; ++s) {
        const int32_t n = recv_count[s] < 0 ? 0 : (recv_count[s] > M ? M : recv_count[s]);
        for (int32_t i = 0; i < n; ++i) {
            const int64_t* row = recv_topk + ((int64_t)s * M + i) * K;
            for (int32_t k = 0; k < K; ++k) {
                const int64_t e = row[k];
                if (e < 0) continue;
                if (e >= E) {
                    status |= ORACLE_BAD_EXPERT;
                    continue;
                }
                if (e < first_expert || e >= first_expert + L) continue;  /* another rank's expert */
                for (int32_t j = 0; j < k; ++j)
                    if (row[j] == e) status |= ORACLE_DUP_EXPERT;
                expert_count[e - first_expert] += 1;
            }
        }
    }

    /* Aligned exclusive prefix sum over the local experts. */
    int64_t run = 0;
    expert_psum[0] = 0;
    for (int32_t e = 0; e < L; ++e) {
        run += align_up(expert_count[e], A);
        expert_psum[e + 1] = (int32_t)run;
    }
    if (expert_psum[L] > recv_capacity) status |= ORACLE_RECV_OVERFLOW;
    if (status) return status;

    /* Slots: a cursor per local expert, walking sources, then rows, then k. */
    int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)L);
    if (!cursor) return ORACLE_BAD_ARGS;
    for (int32_t e = 0; e < L; ++e) cursor[e] = expert_psum[e];
    for (int64_t q = 0; q < expert_psum[L]; ++q) recv_src_row_idx[q] = -1;
    for (int64_t q = 0; q < rows * K; ++q) expert_slot[q] = -1;
    for (int32_t s = 0; s < S; ++s) {
        for (int32_t i = 0; i < recv_count[s]; ++i) {
            const int64_t r = (int64_t)s * M + i;
            for (int32_t k = 0; k < K; ++k) {
                const int64_t e = recv_topk[r * K + k];
                if (e < first_expert || e >= first_expert + L) continue;
                const int64_t slot = cursor[e - first_expert]++;
                expert_slot[r * K + k] = (int32_t)slot;
                recv_src_row_idx[slot] = (int32_t)r;
            }
        }
    }
    free(cursor);
    return 0;
}

int oracle_combine(int64_t num_tokens, int32_t num_topk, int64_t hidden, int64_t rows,
                   const uint16_t* y, const float* weights, const int32_t* expert_slot, double* out) {
    if (num_tokens < 0 || num_topk < 1 || hidden < 0 || rows < 0) return ORACLE_BAD_ARGS;
    for (int64_t t = 0; t < num_tokens; ++t) {
        double* o = out + t * hidden;
        for (int64_t h = 0; h < hidden; ++h) o[h] = 0.0;
        for (int32_t k = 0; k < num_topk; ++k) {
            const int64_t slot = expert_slot[t * num_topk + k];
            if (slot < 0) continue;
            if (slot >= rows) return ORACLE_BAD_ARGS;
            const double w = (double)weights[t * num_topk + k];
            const uint16_t* row = y + slot * hidden;
            for (int64_t h = 0; h < hidden; ++h) o[h] += w * bf16_value(row[h]);
        }
    }
    return 0;
}
