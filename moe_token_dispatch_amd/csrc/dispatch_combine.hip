// Combine on gfx950: bring the expert outputs back to their tokens.
//
// The reverse of the expert-major scatter: out[t] = sum over the token's
// routed k of weight[t, k] * y[expert_slot[t, k]], where y holds one row per
// expert-major slot. The "DeepEP Counting Sort / Bucketization" page keeps the
// slot map for exactly this reuse by the combine kernel (section 6.2); the sum
// itself is the usual top-k weighted mixture. Arithmetic: bf16 rows widened
// to fp32, one fused multiply-add per routed k in ascending k order starting
// from 0, and the fp32 sum rounded to bf16 to nearest, ties to even.
//
// One wavefront per (token, row segment of up to 64 x V 16-byte vectors, i.e.
// 8 bf16 per lane-vector) keeps its segment's sums in registers, gathers the
// token's K expert rows (wavefront-uniform slots and weights, read once into
// scalar registers through readlane) and writes the segment once. The kernel
// reads about K rows per token and writes one, so it is bound by HBM reads.
#include "dispatch_common.hpp"

namespace moe_dispatch {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCombineWaves = 4;
constexpr int kCombineMaxVecs = 8;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kStreamingPolicy = 2 | 16;  // nt | sc1

struct CombineParams {
    int64_t num_tokens;
    int64_t row_vecs;      // 16-byte vectors per row (hidden / 8)
    int64_t expert_rows;   // rows of y
    int64_t token_waves;   // num_tokens * segments, rounded up to whole workgroups
    int32_t num_topk;
    int32_t segments;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int V>
__global__ void __launch_bounds__(kCombineWaves * kWave)
combine_kernel(const u32x4* __restrict__ y, const float* __restrict__ weights,
               const int32_t* __restrict__ expert_slot, CombineParams p, u32x4* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave_id = (int64_t)blockIdx.x * kCombineWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (wave_id >= p.num_tokens * p.segments) return;
    const int64_t t = wave_id / p.segments;
    const int seg = (int)(wave_id - t * p.segments);
    const int K = p.num_topk;
    int slot = -1;
    float w = 0.f;
    if (lane < K) {
        slot = expert_slot[t * K + lane];
        w = weights[t * K + lane];
    }
    // A slot outside y never occurs for a layout with status 0; it is dropped.
    if (slot >= p.expert_rows) slot = -1;

    const int64_t nv = p.row_vecs;
    const int64_t base = (int64_t)seg * kWave * V;
    float acc[V][8];
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[j][q] = 0.f;

    for (int k = 0; k < K; ++k) {
        const int s = __builtin_amdgcn_readlane(slot, k);
        if (s < 0) continue;
        const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w), k));
        const u32x4* row = y + (int64_t)s * nv;
        u32x4 v[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int64_t i = base + j * kWave + lane;
            v[j] = i < nv ? row[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < V; ++j) {
            acc[j][0] = __builtin_fmaf(wk, bf16_lo(v[j].x), acc[j][0]);
            acc[j][1] = __builtin_fmaf(wk, bf16_hi(v[j].x), acc[j][1]);
            acc[j][2] = __builtin_fmaf(wk, bf16_lo(v[j].y), acc[j][2]);
            acc[j][3] = __builtin_fmaf(wk, bf16_hi(v[j].y), acc[j][3]);
            acc[j][4] = __builtin_fmaf(wk, bf16_lo(v[j].z), acc[j][4]);
            acc[j][5] = __builtin_fmaf(wk, bf16_hi(v[j].z), acc[j][5]);
            acc[j][6] = __builtin_fmaf(wk, bf16_lo(v[j].w), acc[j][6]);
            acc[j][7] = __builtin_fmaf(wk, bf16_hi(v[j].w), acc[j][7]);
        }
    }

    // One row per token; vectors past the row end fall outside the row's
    // buffer range and are dropped by the hardware.
    const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(out + t * nv, 0, (int)(nv * 16), kBufferWord3);
#pragma unroll
    for (int j = 0; j < V; ++j) {
        u32x4 o;
        o.x = to_bf16(acc[j][0]) | (to_bf16(acc[j][1]) << 16);
        o.y = to_bf16(acc[j][2]) | (to_bf16(acc[j][3]) << 16);
        o.z = to_bf16(acc[j][4]) | (to_bf16(acc[j][5]) << 16);
        o.w = to_bf16(acc[j][6]) | (to_bf16(acc[j][7]) << 16);
        __builtin_amdgcn_raw_buffer_store_b128(o, dst, (int)((base + j * kWave + lane) * 16), 0, kStreamingPolicy);
    }
}

template <int V>
hipError_t launch_v(dim3 grid, hipStream_t stream, const u32x4* y, const float* weights, const int32_t* slots,
                    CombineParams p, u32x4* out) {
    void* args[] = {&y, &weights, &slots, &p, &out};
    return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel<V>), grid, dim3(kCombineWaves * kWave),
                           args, 0, stream);
}

}  // namespace

hipError_t launch_combine(int64_t num_tokens, int32_t num_topk, int64_t row_bytes, int64_t expert_rows,
                          const int32_t* expert_slot, const float* weights, const void* y, void* out,
                          hipStream_t stream) {
    CombineParams p{};
    p.num_tokens = num_tokens;
    p.row_vecs = row_bytes / 16;
    p.expert_rows = expert_rows;
    p.num_topk = num_topk;
    p.segments = (int32_t)((p.row_vecs + kWave * kCombineMaxVecs - 1) / (kWave * kCombineMaxVecs));
    if (p.segments < 1) p.segments = 1;
    const int64_t seg_vecs = (p.row_vecs + p.segments - 1) / p.segments;
    const int v = (int)((seg_vecs + kWave - 1) / kWave);
    const int64_t waves = num_tokens * p.segments;
    p.token_waves = (waves + kCombineWaves - 1) / kCombineWaves * kCombineWaves;
    const int64_t blocks = p.token_waves / kCombineWaves;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks);
    const auto* ys = static_cast<const u32x4*>(y);
    auto* os = static_cast<u32x4*>(out);
    switch (v) {
        case 1: return launch_v<1>(grid, stream, ys, weights, expert_slot, p, os);
        case 2: return launch_v<2>(grid, stream, ys, weights, expert_slot, p, os);
        case 3: return launch_v<3>(grid, stream, ys, weights, expert_slot, p, os);
        case 4: return launch_v<4>(grid, stream, ys, weights, expert_slot, p, os);
        case 5: return launch_v<5>(grid, stream, ys, weights, expert_slot, p, os);
        case 6: return launch_v<6>(grid, stream, ys, weights, expert_slot, p, os);
        case 7: return launch_v<7>(grid, stream, ys, weights, expert_slot, p, os);
        default: return launch_v<8>(grid, stream, ys, weights, expert_slot, p, os);
    }
}

}  // namespace moe_dispatch
