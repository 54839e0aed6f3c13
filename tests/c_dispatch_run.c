/* One dispatch driven from C alone: buffers from hipMalloc, no Python or torch
 * in the process. Built by tests/c_programs.py, run by tests/test_gpu_c_caller.py.
 *
 * Reads the problem and its inputs from the file argv[1]:
 *   int64 T, K, E, R, A, row_bytes, S, one_call;
 *   int64 topk_idx[T*K]; uint8 x[T*row_bytes]; float x_sf[T*S].
 * Fills every output buffer with 0xA5 bytes, runs dispatch_layout then
 * dispatch_scatter (or dispatch_layout_and_scatter when one_call is set) with
 * every output selected and worst-case capacities, on a stream of its own, and
 * writes to the file argv[2]:
 *   int32 return code; int64 recv_capacity, rank_capacity;
 *   int32 status, expert_count[E], rank_count[R], expert_psum[E+1],
 *   rank_psum[R+1], expert_slot[T*K], rank_slot[T*K],
 *   recv_src_token_idx[recv_capacity], rank_src_token_idx[rank_capacity];
 *   uint8 rank_x[rank_capacity*row_bytes]; float rank_sf[rank_capacity*S];
 *   uint8 recv_x[recv_capacity*row_bytes]; float recv_sf[recv_capacity*S].
 * Exit status 0 when every HIP call succeeded (the return code is in the file). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_dispatch.h"

#define HIP_OK(call)                                                                    \
    do {                                                                                \
        hipError_t err_ = (call);                                                       \
        if (err_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(err_));          \
            exit(2);                                                                    \
        }                                                                               \
    } while (0)

static void* dev_filled(size_t bytes) {
    void* p = NULL;
    const size_t n = bytes ? bytes : 16;
    HIP_OK(hipMalloc(&p, n));
    HIP_OK(hipMemset(p, 0xA5, n));
    return p;
}

static void* host_read(FILE* f, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p || (bytes && fread(p, 1, bytes, f) != bytes)) {
        fprintf(stderr, "short input\n");
        exit(3);
    }
    return p;
}

static void put_dev(FILE* f, const void* d, size_t bytes) {
    if (!bytes) return;
    void* h = malloc(bytes);
    if (!h) exit(3);
    HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    if (fwrite(h, 1, bytes, f) != bytes) exit(3);
    free(h);
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s input output\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 1;
    int64_t hdr[8];
    if (fread(hdr, sizeof hdr, 1, in) != 1) return 3;
    const int64_t T = hdr[0], K = hdr[1], E = hdr[2], R = hdr[3], A = hdr[4], RB = hdr[5], S = hdr[6];
    const int one_call = hdr[7] != 0;

    dispatch_problem_t p;
    memset(&p, 0, sizeof p);
    p.num_tokens = T;
    p.num_topk = (int32_t)K;
    p.num_experts = (int32_t)E;
    p.num_ranks = (int32_t)R;
    p.expert_alignment = (int32_t)A;
    p.topk_idx_bytes = 8;
    p.sf_per_token = (int32_t)S;
    p.row_bytes = RB;
    p.flags = DISPATCH_ALL_OUTPUTS;
    int64_t recv_cap = 0, rank_cap = 0;
    int rc = dispatch_max_rows(&p, &recv_cap, &rank_cap);
    p.recv_capacity_rows = recv_cap;
    p.rank_capacity_rows = rank_cap;
    size_t ws_bytes = 0;
    if (rc == 0) rc = dispatch_workspace_size(&p, &ws_bytes);
    if (rc != 0) {
        fprintf(stderr, "host error %d: %s\n", rc, dispatch_strerror(rc));
        return 4;
    }

    const size_t topk_bytes = (size_t)(T * K) * 8, x_bytes = (size_t)(T * RB), sf_bytes = (size_t)(T * S) * 4;
    void* h_topk = host_read(in, topk_bytes);
    void* h_x = host_read(in, x_bytes);
    void* h_sf = host_read(in, sf_bytes);
    fclose(in);

    void* d_topk = dev_filled(topk_bytes);
    void* d_x = dev_filled(x_bytes);
    void* d_sf = S ? dev_filled(sf_bytes) : NULL;
    HIP_OK(hipMemcpy(d_topk, h_topk, topk_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, h_x, x_bytes, hipMemcpyHostToDevice));
    if (S) HIP_OK(hipMemcpy(d_sf, h_sf, sf_bytes, hipMemcpyHostToDevice));

    dispatch_layout_t lay;
    memset(&lay, 0, sizeof lay);
    lay.status = dev_filled(4);
    lay.expert_count = dev_filled((size_t)E * 4);
    lay.rank_count = dev_filled((size_t)R * 4);
    lay.expert_psum = dev_filled((size_t)(E + 1) * 4);
    lay.rank_psum = dev_filled((size_t)(R + 1) * 4);
    lay.expert_slot = dev_filled((size_t)(T * K) * 4);
    lay.rank_slot = dev_filled((size_t)(T * K) * 4);
    lay.recv_src_token_idx = dev_filled((size_t)recv_cap * 4);
    lay.rank_src_token_idx = dev_filled((size_t)rank_cap * 4);
    void* rank_x = dev_filled((size_t)(rank_cap * RB));
    float* rank_sf = S ? dev_filled((size_t)(rank_cap * S) * 4) : NULL;
    void* recv_x = dev_filled((size_t)(recv_cap * RB));
    float* recv_sf = S ? dev_filled((size_t)(recv_cap * S) * 4) : NULL;
    void* ws = dev_filled(ws_bytes);
    HIP_OK(hipDeviceSynchronize());

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    if (one_call) {
        rc = dispatch_layout_and_scatter(&p, d_topk, &lay, ws, ws_bytes, d_x, d_sf, rank_x, rank_sf, recv_x, recv_sf,
                                         stream);
    } else {
        rc = dispatch_layout(&p, d_topk, &lay, ws, ws_bytes, stream);
        if (rc == 0) rc = dispatch_scatter(&p, &lay, d_x, d_sf, rank_x, rank_sf, recv_x, recv_sf, stream);
    }
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipStreamDestroy(stream));

    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    const int32_t rc32 = rc;
    fwrite(&rc32, 4, 1, out);
    fwrite(&recv_cap, 8, 1, out);
    fwrite(&rank_cap, 8, 1, out);
    put_dev(out, lay.status, 4);
    put_dev(out, lay.expert_count, (size_t)E * 4);
    put_dev(out, lay.rank_count, (size_t)R * 4);
    put_dev(out, lay.expert_psum, (size_t)(E + 1) * 4);
    put_dev(out, lay.rank_psum, (size_t)(R + 1) * 4);
    put_dev(out, lay.expert_slot, (size_t)(T * K) * 4);
    put_dev(out, lay.rank_slot, (size_t)(T * K) * 4);
    put_dev(out, lay.recv_src_token_idx, (size_t)recv_cap * 4);
    put_dev(out, lay.rank_src_token_idx, (size_t)rank_cap * 4);
    put_dev(out, rank_x, (size_t)(rank_cap * RB));
    if (S) put_dev(out, rank_sf, (size_t)(rank_cap * S) * 4);
    put_dev(out, recv_x, (size_t)(recv_cap * RB));
    if (S) put_dev(out, recv_sf, (size_t)(recv_cap * S) * 4);
    fclose(out);

    void* bufs[] = {d_topk, d_x, d_sf, lay.status, lay.expert_count, lay.rank_count, lay.expert_psum,
                    lay.rank_psum, lay.expert_slot, lay.rank_slot, lay.recv_src_token_idx,
                    lay.rank_src_token_idx, rank_x, rank_sf, recv_x, recv_sf, ws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i]) HIP_OK(hipFree(bufs[i]));
    free(h_topk);
    free(h_x);
    free(h_sf);
    return 0;
}
