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
// One wavefront per (token, 1 KB row segment: one 16-byte vector of 8 bf16 per
// lane) keeps its segment's sums in registers. It issues the loads of up to
// eight of the token's expert rows before the first multiply-add, so a
// wavefront has 8 KB of independent reads in flight, and writes its segment
// once. The kernel reads about K rows per token and writes one: it is bound by
// HBM reads. Every y row is read once per launch, so the loads are marked
// nontemporal; the output goes out with the sc1 policy (measured best for
// this kernel among the store policies).
#include "dispatch_common.hpp"
#include "dispatch_device.hpp"

namespace moe_dispatch {
namespace {

constexpr int kCombineWaves = 2;         // wavefronts per workgroup
constexpr int kCombineBatch = 8;         // expert rows loaded before the multiply-adds
constexpr int64_t kMaxCombineBlocks = int64_t(1) << 16;  // larger grids loop

struct CombineParams {
    int64_t num_tokens;
    int64_t row_vecs;      // 16-byte vectors per row (hidden / 8)
    int64_t expert_rows;   // rows of y
    int64_t total_waves;   // num_tokens * segments
    int64_t wave_stride;   // wavefronts in the grid
    int32_t num_topk;
    int32_t segments;      // row segments of kWave vectors
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ void __launch_bounds__(kCombineWaves * kWave)
combine_kernel(const u32x4* __restrict__ y, const float* __restrict__ weights,
               const int32_t* __restrict__ expert_slot, CombineParams p, u32x4* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int K = p.num_topk;
    const int64_t nv = p.row_vecs;
    for (int64_t wave_id = (int64_t)blockIdx.x * kCombineWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
         wave_id < p.total_waves; wave_id += p.wave_stride) {
        const int64_t t = wave_id / p.segments;
        const int64_t i = (wave_id - t * p.segments) * kWave + lane;  // this lane's vector in the row
        const bool live = i < nv;
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        for (int k0 = 0; k0 < K; k0 += kCombineBatch) {
            // Lane b of the batch holds entry k0 + b of the token.
            int slot = -1;
            float w = 0.f;
            if (lane < kCombineBatch && k0 + lane < K) {
                slot = expert_slot[t * K + k0 + lane];
                w = weights[t * K + k0 + lane];
            }
            // A slot outside y never occurs for a layout with status 0; it is dropped.
            if (slot >= p.expert_rows) slot = -1;
            int s[kCombineBatch];
            u32x4 v[kCombineBatch];
#pragma unroll
            for (int b = 0; b < kCombineBatch; ++b) {
                s[b] = __builtin_amdgcn_readlane(slot, b);
                v[b] = u32x4{0u, 0u, 0u, 0u};
                if (s[b] >= 0 && live) v[b] = __builtin_nontemporal_load(y + (int64_t)s[b] * nv + i);
            }
#pragma unroll
            for (int b = 0; b < kCombineBatch; ++b) {
                if (s[b] < 0) continue;
                const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w), b));
                acc[0] = __builtin_fmaf(wk, bf16_lo(v[b].x), acc[0]);
                acc[1] = __builtin_fmaf(wk, bf16_hi(v[b].x), acc[1]);
                acc[2] = __builtin_fmaf(wk, bf16_lo(v[b].y), acc[2]);
                acc[3] = __builtin_fmaf(wk, bf16_hi(v[b].y), acc[3]);
                acc[4] = __builtin_fmaf(wk, bf16_lo(v[b].z), acc[4]);
                acc[5] = __builtin_fmaf(wk, bf16_hi(v[b].z), acc[5]);
                acc[6] = __builtin_fmaf(wk, bf16_lo(v[b].w), acc[6]);
                acc[7] = __builtin_fmaf(wk, bf16_hi(v[b].w), acc[7]);
            }
        }
        // One row per token; a vector past the row end falls outside the
        // row's buffer range and is dropped by the hardware.
        const RowStore<kSc1Policy> dst(out + t * nv, (int)(nv * 16));
        u32x4 o;
        o.x = to_bf16(acc[0]) | (to_bf16(acc[1]) << 16);
        o.y = to_bf16(acc[2]) | (to_bf16(acc[3]) << 16);
        o.z = to_bf16(acc[4]) | (to_bf16(acc[5]) << 16);
        o.w = to_bf16(acc[6]) | (to_bf16(acc[7]) << 16);
        dst.store(live ? i : nv, o);
    }
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
    p.segments = (int32_t)((p.row_vecs + kWave - 1) / kWave);
    p.total_waves = num_tokens * p.segments;
    int64_t blocks = (p.total_waves + kCombineWaves - 1) / kCombineWaves;
    if (blocks == 0) return hipSuccess;
    if (blocks > kMaxCombineBlocks) blocks = kMaxCombineBlocks;
    p.wave_stride = blocks * kCombineWaves;
    const auto* ys = static_cast<const u32x4*>(y);
    auto* os = static_cast<u32x4*>(out);
    void* args[] = {&ys, &weights, &expert_slot, &p, &os};
    return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), dim3((unsigned)blocks),
                           dim3(kCombineWaves * kWave), args, 0, stream);
}

}  // namespace moe_dispatch
