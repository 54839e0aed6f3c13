/* The library driven from C alone: buffers from hipMalloc, no Python or torch
 * in the process. Built by tests/c_programs.py, run by tests/test_gpu_c_caller.py
 * as `c_dispatch_run MODE input output`, MODE one of dispatch, expand, combine.
 * Every output buffer is filled with 0xA5 bytes before the calls (the
 * workspaces are zero-filled, as the ABI asks), which run on
 * a stream of their own with worst-case capacities; every output buffer is
 * then written to the output file. Exit status 0 when every HIP call
 * succeeded (the library's return code is the first field of the output).
 *
 * dispatch  in:  int64 T, K, E, R, A, row_bytes, S, one_call;
 *                int64 topk_idx[T*K]; uint8 x[T*row_bytes]; float x_sf[T*S].
 *           out: int32 rc; int64 recv_capacity, rank_capacity; int32 status,
 *                expert_count[E], rank_count[R], expert_psum[E+1],
 *                rank_psum[R+1], expert_slot[T*K], rank_slot[T*K],
 *                recv_src_token_idx[recv_capacity],
 *                rank_src_token_idx[rank_capacity]; uint8 rank_x[..];
 *                float rank_sf[..]; uint8 recv_x[..]; float recv_sf[..].
 *           dispatch_layout + dispatch_scatter, or dispatch_layout_and_scatter.
 * expand    in:  int64 S, M, K, E, R, local_rank, A, row_bytes, SF, one_call;
 *                int64 recv_topk_idx[S*M*K]; int32 recv_count[S];
 *                uint8 recv_buf[S*M*row_bytes]; float recv_sf_buf[S*M*SF].
 *           out: int32 rc; int64 recv_capacity; int32 status,
 *                expert_count[E/R], expert_psum[E/R+1], expert_slot[S*M*K],
 *                recv_src_row_idx[recv_capacity]; uint8 recv_x[..];
 *                float recv_sf[..].
 *           dispatch_expand_layout + dispatch_expand_scatter, or
 *           dispatch_expand_layout_and_scatter.
 * combine   in:  int64 T, K, H, expert_rows; int32 expert_slot[T*K];
 *                float topk_weights[T*K]; uint16 y[expert_rows*H] (bf16 bits).
 *           out: int32 rc; uint16 out[T*H] (bf16 bits). */
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

/* A workspace: zero-filled before its first use, as the ABI asks. */
static void* dev_zeroed(size_t bytes) {
    void* p = NULL;
    const size_t n = bytes ? bytes : 16;
    HIP_OK(hipMalloc(&p, n));
    HIP_OK(hipMemset(p, 0, n));
    return p;
}

/* Reads `bytes` from the input into a new device buffer. */
static void* dev_read(FILE* f, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    if (!h || (bytes && fread(h, 1, bytes, f) != bytes)) {
        fprintf(stderr, "short input\n");
        exit(3);
    }
    void* d = dev_filled(bytes);
    if (bytes) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    free(h);
    return d;
}

static void put(FILE* f, const void* h, size_t bytes) {
    if (bytes && fwrite(h, 1, bytes, f) != bytes) exit(3);
}

static void put_dev(FILE* f, const void* d, size_t bytes) {
    if (!bytes) return;
    void* h = malloc(bytes);
    if (!h) exit(3);
    HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    put(f, h, bytes);
    free(h);
}

static void read_header(FILE* f, int64_t* hdr, size_t n) {
    if (fread(hdr, sizeof(int64_t), n, f) != n) {
        fprintf(stderr, "short header\n");
        exit(3);
    }
}

static void host_error(int rc) {
    fprintf(stderr, "host error %d: %s\n", rc, dispatch_strerror(rc));
    exit(4);
}

static int run_dispatch(FILE* in, FILE* out, hipStream_t stream) {
    int64_t h[8];
    read_header(in, h, 8);
    const int64_t T = h[0], K = h[1], E = h[2], R = h[3], A = h[4], RB = h[5], S = h[6];
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
    if (rc) host_error(rc);
    p.recv_capacity_rows = recv_cap;
    p.rank_capacity_rows = rank_cap;
    size_t ws_bytes = 0;
    rc = dispatch_workspace_size(&p, &ws_bytes);
    if (rc) host_error(rc);

    void* topk = dev_read(in, (size_t)(T * K) * 8);
    void* x = dev_read(in, (size_t)(T * RB));
    float* x_sf = S ? dev_read(in, (size_t)(T * S) * 4) : NULL;
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
    void* ws = dev_zeroed(ws_bytes);
    HIP_OK(hipDeviceSynchronize());

    if (h[7]) {
        rc = dispatch_layout_and_scatter(&p, topk, &lay, ws, ws_bytes, x, x_sf, rank_x, rank_sf, recv_x, recv_sf,
                                         stream);
    } else {
        rc = dispatch_layout(&p, topk, &lay, ws, ws_bytes, stream);
        if (rc == 0) rc = dispatch_scatter(&p, &lay, x, x_sf, rank_x, rank_sf, recv_x, recv_sf, stream);
    }
    HIP_OK(hipStreamSynchronize(stream));

    const int32_t rc32 = rc;
    put(out, &rc32, 4);
    put(out, &recv_cap, 8);
    put(out, &rank_cap, 8);
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

    void* bufs[] = {topk, x, x_sf, lay.status, lay.expert_count, lay.rank_count, lay.expert_psum, lay.rank_psum,
                    lay.expert_slot, lay.rank_slot, lay.recv_src_token_idx, lay.rank_src_token_idx, rank_x,
                    rank_sf, recv_x, recv_sf, ws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i]) HIP_OK(hipFree(bufs[i]));
    return 0;
}

static int run_expand(FILE* in, FILE* out, hipStream_t stream) {
    int64_t h[10];
    read_header(in, h, 10);
    const int64_t S = h[0], M = h[1], K = h[2], E = h[3], R = h[4], RB = h[7], SF = h[8];
    const int64_t EL = E / R, rows = S * M;
    dispatch_expand_problem_t q;
    memset(&q, 0, sizeof q);
    q.num_sources = (int32_t)S;
    q.rows_per_source = (int32_t)M;
    q.num_topk = (int32_t)K;
    q.num_experts = (int32_t)E;
    q.num_ranks = (int32_t)R;
    q.local_rank = (int32_t)h[5];
    q.expert_alignment = (int32_t)h[6];
    q.topk_idx_bytes = 8;
    q.sf_per_token = (int32_t)SF;
    q.row_bytes = RB;
    int64_t recv_cap = 0;
    int rc = dispatch_expand_max_rows(&q, &recv_cap);
    if (rc) host_error(rc);
    q.recv_capacity_rows = recv_cap;
    size_t ws_bytes = 0;
    rc = dispatch_expand_workspace_size(&q, &ws_bytes);
    if (rc) host_error(rc);

    void* topk = dev_read(in, (size_t)(rows * K) * 8);
    int32_t* counts = dev_read(in, (size_t)S * 4);
    void* buf = dev_read(in, (size_t)(rows * RB));
    float* buf_sf = SF ? dev_read(in, (size_t)(rows * SF) * 4) : NULL;
    dispatch_layout_t lay;
    memset(&lay, 0, sizeof lay);  /* the rank fields stay NULL */
    lay.status = dev_filled(4);
    lay.expert_count = dev_filled((size_t)EL * 4);
    lay.expert_psum = dev_filled((size_t)(EL + 1) * 4);
    lay.expert_slot = dev_filled((size_t)(rows * K) * 4);
    lay.recv_src_token_idx = dev_filled((size_t)recv_cap * 4);
    void* recv_x = dev_filled((size_t)(recv_cap * RB));
    float* recv_sf = SF ? dev_filled((size_t)(recv_cap * SF) * 4) : NULL;
    void* ws = dev_zeroed(ws_bytes);
    HIP_OK(hipDeviceSynchronize());

    if (h[9]) {
        rc = dispatch_expand_layout_and_scatter(&q, topk, counts, &lay, ws, ws_bytes, buf, buf_sf, recv_x, recv_sf,
                                                stream);
    } else {
        rc = dispatch_expand_layout(&q, topk, counts, &lay, ws, ws_bytes, stream);
        if (rc == 0) rc = dispatch_expand_scatter(&q, &lay, buf, buf_sf, recv_x, recv_sf, stream);
    }
    HIP_OK(hipStreamSynchronize(stream));

    const int32_t rc32 = rc;
    put(out, &rc32, 4);
    put(out, &recv_cap, 8);
    put_dev(out, lay.status, 4);
    put_dev(out, lay.expert_count, (size_t)EL * 4);
    put_dev(out, lay.expert_psum, (size_t)(EL + 1) * 4);
    put_dev(out, lay.expert_slot, (size_t)(rows * K) * 4);
    put_dev(out, lay.recv_src_token_idx, (size_t)recv_cap * 4);
    put_dev(out, recv_x, (size_t)(recv_cap * RB));
    if (SF) put_dev(out, recv_sf, (size_t)(recv_cap * SF) * 4);

    void* bufs[] = {topk, counts, buf, buf_sf, lay.status, lay.expert_count, lay.expert_psum, lay.expert_slot,
                    lay.recv_src_token_idx, recv_x, recv_sf, ws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i]) HIP_OK(hipFree(bufs[i]));
    return 0;
}

static int run_combine(FILE* in, FILE* out, hipStream_t stream) {
    int64_t h[4];
    read_header(in, h, 4);
    const int64_t T = h[0], K = h[1], H = h[2], Y = h[3];
    dispatch_combine_problem_t c;
    memset(&c, 0, sizeof c);
    c.num_tokens = T;
    c.num_topk = (int32_t)K;
    c.hidden = H;
    c.expert_rows = Y;
    int32_t* slots = dev_read(in, (size_t)(T * K) * 4);
    float* weights = dev_read(in, (size_t)(T * K) * 4);
    void* y = dev_read(in, (size_t)(Y * H) * 2);
    void* o = dev_filled((size_t)(T * H) * 2);
    HIP_OK(hipDeviceSynchronize());
    const int rc = dispatch_combine(&c, slots, weights, y, o, stream);
    HIP_OK(hipStreamSynchronize(stream));
    const int32_t rc32 = rc;
    put(out, &rc32, 4);
    put_dev(out, o, (size_t)(T * H) * 2);
    void* bufs[] = {slots, weights, y, o};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 4) {
        fprintf(stderr, "usage: %s dispatch|expand|combine input output\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[2], "rb");
    FILE* out = fopen(argv[3], "wb");
    if (!in || !out) return 1;
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    int rc;
    if (strcmp(argv[1], "dispatch") == 0)
        rc = run_dispatch(in, out, stream);
    else if (strcmp(argv[1], "expand") == 0)
        rc = run_expand(in, out, stream);
    else if (strcmp(argv[1], "combine") == 0)
        rc = run_combine(in, out, stream);
    else
        rc = 1;
    HIP_OK(hipStreamDestroy(stream));
    fclose(in);
    if (fclose(out) != 0) return 3;
    return rc;
}
