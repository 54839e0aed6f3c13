// Row scatter on gfx950: copy each token row into its rank-contiguous rows and
// its expert-major rows, and zero the alignment pad rows.
//
// This is the data move of the method ("DeepEP Counting Sort / Bucketization"
// page): the rank-level copy of sections 6.2-6.3, the expert-major copy of the
// expand mode (sections 6.4 and 8.2) and the zero padding of section 7.3. It
// moves nearly all of the bytes, so it is built for HBM bandwidth. Two
// kernels, chosen per problem by the launcher:
//  - split_scatter_kernel (a dispatch whose rows were just read into the
//    Infinity Cache): a token row is cut into 1 KB segments; one workgroup per
//    (token, segment), whose wavefronts each read the segment, 16 bytes per
//    lane per instruction, and write it to their share of the token's
//    destination rows, with the workgroups per CU bounded;
//  - scatter_kernel (rows from HBM, and rows with about one destination: the
//    receiver-side expand, a top-1 copy): one wavefront per (token, segment of
//    1 KB, or 4 KB with about one destination) reads its segment once and
//    writes it to every destination.
// Both are the read-once / write-to-many-destinations copy of the "Symmetric
// Memory" page's sender warp, here to local rows.
// Destination slots are wavefront-uniform (readlane), so destination loops
// run on scalar registers. Pad rows are cleared by extra wavefronts after the
// token workgroups: one row each in scatter_kernel, 4 KB of a row each in
// split_scatter_kernel.
//
// Row stores go through a buffer resource that spans exactly one destination
// row, so the hardware drops any offset outside that row, and carry the
// streaming cache policy (nt with sc1): the output is far larger than the
// caches and is not read back here, and of the store forms measured on MI355X
// this one moved the rows fastest. Walking the destinations instead (each
// destination row written by consecutive workgroups, its source row read
// once per destination from the Infinity Cache) measured slower than the
// split kernel with bounded occupancy on every batch tried (7 KB fp8 rows:
// 97.7 against 94.6 us; 8 KB bf16 rows of 16384 tokens: 351 against 306 us).
#include "dispatch_common.hpp"
#include "dispatch_device.hpp"

namespace moe_dispatch {
namespace {

static_assert(DISPATCH_MAX_EXPERTS <= kWave * kWave, "expert_of_row searches two rounds of 64 samples");
// V, the 16-byte vectors per lane of one row segment, and W, the wavefronts
// per workgroup, follow the stores per loaded row (measured on MI355X): with
// many destinations per row (dispatch: K expert rows and the rank rows) one
// vector per lane in one-wavefront workgroups, i.e. many short wavefronts,
// moves the rows fastest (65536 x 7 KB fp8 tokens from HBM: 1198 us against
// 1223 us with four wavefronts per workgroup); with about one destination per
// row (the receiver-side expand, a top-1 copy) four vectors per lane in
// four-wavefront workgroups do.
constexpr int kVecsManyDestinations = 1;
constexpr int kWavesManyDestinations = 1;
constexpr int kVecsFewDestinations = 4;
constexpr int kWavesFewDestinations = 4;

struct ScatterParams {
    int64_t num_tokens;
    int64_t row_vecs;        // row_bytes / 16
    int64_t token_waves;     // num_tokens * segments, rounded up to whole workgroups
    int64_t recv_capacity;   // rows of recv_x / recv_sf
    int64_t rank_capacity;   // rows of rank_x / rank_sf
    int32_t num_topk;
    int32_t segments;        // row segments per token
    int32_t sf_per_token;
    int32_t num_experts;
    int32_t pad_waves_per_expert;  // pad rows per expert covered: alignment - 1 with pads, else 1
    int32_t pad_parts;             // wavefronts per pad row, each zeroing pad_part_vecs vectors
    int64_t pad_part_vecs;
    int32_t pad_by_block;          // pad wavefronts mapped per row block (else per expert)
    int32_t alignment;
    int32_t write_rank;      // rank_x / rank_sf requested
    int32_t write_expert;    // recv_x / recv_sf requested
    int64_t token_groups;    // split kernel: workgroups of token segments (num_tokens * segments)
};

template <int V>
__device__ __forceinline__ void copy_token(const u32x4* __restrict__ x, const uint32_t* __restrict__ x_sf,
                                           const ScatterParams& p, int64_t t, int seg, int lane,
                                           const int32_t* __restrict__ expert_slot,
                                           const int32_t* __restrict__ rank_slot,
                                           u32x4* __restrict__ rank_x, uint32_t* __restrict__ rank_sf,
                                           u32x4* __restrict__ recv_x, uint32_t* __restrict__ recv_sf,
                                           const int32_t* __restrict__ status) {
    const int K = p.num_topk;
    // The status and the token's slots are loaded together; a non-zero
    // status (an unspecified layout) writes nothing.
    const int st = *status;
    int es = -1, rs = -1;
    if (lane < K) {
        es = expert_slot[t * K + lane];
        rs = rank_slot != nullptr ? rank_slot[t * K + lane] : -1;
    }
    asm volatile("" ::: "memory");  // the loads go out before the check below
    if (st != 0) return;
    // Slots past the capacities never occur for a layout with status 0; they
    // are dropped here so that no store can leave the output buffers.
    if (!p.write_expert || es >= p.recv_capacity) es = -1;
    if (!p.write_rank || rs >= p.rank_capacity) rs = -1;
    // A row with no destination (fully masked token, unused receive-buffer
    // row) is not read at all.
    if (__ballot(es >= 0 || rs >= 0) == 0ull) return;
    const int64_t nv = p.row_vecs;
    const u32x4* src = x + t * nv;
    {
        const int64_t base = (int64_t)seg * kWave * V;
        u32x4 v[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int64_t i = base + j * kWave + lane;
            if (i < nv) v[j] = src[i];
        }
        for (int k = 0; k < K; ++k) {
            // Vectors past the row end fall outside the row's buffer range and are dropped.
            const int d_expert = __builtin_amdgcn_readlane(es, k);
            if (d_expert >= 0) {
                const RowWriter dst(recv_x + (int64_t)d_expert * nv, (int)(nv * 16));
#pragma unroll
                for (int j = 0; j < V; ++j) dst.store(base + j * kWave + lane, v[j]);
            }
            const int d_rank = __builtin_amdgcn_readlane(rs, k);
            if (d_rank >= 0) {
                const RowWriter dst(rank_x + (int64_t)d_rank * nv, (int)(nv * 16));
#pragma unroll
                for (int j = 0; j < V; ++j) dst.store(base + j * kWave + lane, v[j]);
            }
        }
    }
    const int S = seg == 0 ? p.sf_per_token : 0;  // the first segment's wavefront moves the scale factors
    for (int s0 = 0; s0 < S; s0 += kWave) {
        const int i = s0 + lane;
        const uint32_t v = i < S ? x_sf[t * S + i] : 0u;
        for (int k = 0; k < K; ++k) {
            const int d_expert = __builtin_amdgcn_readlane(es, k);
            if (d_expert >= 0 && i < S) recv_sf[(int64_t)d_expert * S + i] = v;
            const int d_rank = __builtin_amdgcn_readlane(rs, k);
            if (d_rank >= 0 && i < S) rank_sf[(int64_t)d_rank * S + i] = v;
        }
    }
}

// The expert whose receive rows hold `row`: the largest e with
// expert_psum[e] <= row, found by the whole wavefront in two rounds over the
// non-decreasing psums (64 evenly spaced samples, then the chunk between two
// samples), since E <= 64 * 64. -1 if expert_psum[0] > row (never for a
// valid layout, whose psums start at 0).
__device__ __forceinline__ int expert_of_row(int64_t row, int num_experts, int lane,
                                             const int32_t* __restrict__ expert_psum) {
    const int step = (num_experts + kWave - 1) / kWave;
    const int i1 = lane * step;
    const int c1 = __popcll(__ballot(i1 < num_experts && expert_psum[i1] <= row));
    if (c1 == 0) return -1;
    const int base = (c1 - 1) * step;
    const int i2 = base + lane;
    return base + __popcll(__ballot(lane < step && i2 < num_experts && expert_psum[i2] <= row)) - 1;
}

// Pad rows (section 7.3): the rows after an expert's routed rows up to its
// aligned end, at most alignment - 1 of them, all in the expert's last
// block of `alignment` rows (the aligned psums are multiples of it). One
// wavefront zeroes one row, under one of two mappings; the launcher takes the
// one with fewer wavefronts:
//  - per expert: wavefront (e, j) zeroes the j-th pad row of expert e;
//  - per block: wavefront (b, j) zeroes row b * alignment + 1 + j if block b
//    is the last of its expert and that row is past the expert's routed rows.
//    Routed rows span at most min(E, T*K) + T*K / alignment blocks, far fewer
//    than E experts when the batch is small: then most per-expert wavefronts
//    would find no pad row and only cost their launch.
__device__ __forceinline__ void zero_pads(const ScatterParams& p, int64_t pad_wave, int lane,
                                          const int32_t* __restrict__ expert_count,
                                          const int32_t* __restrict__ expert_psum,
                                          u32x4* __restrict__ recv_x, uint32_t* __restrict__ recv_sf) {
    // A pad row is zeroed by pad_parts consecutive wavefronts, pad_part_vecs
    // vectors each.
    const int64_t row_wave = pad_wave / p.pad_parts;
    const int part = (int)(pad_wave - row_wave * p.pad_parts);
    pad_wave = row_wave;
    int64_t row;
    int e;
    if (p.pad_by_block) {
        const int64_t b = pad_wave / p.pad_waves_per_expert;
        const int64_t block0 = b * p.alignment;
        e = expert_of_row(block0, p.num_experts, lane, expert_psum);
        if (e < 0 || expert_psum[e + 1] != block0 + p.alignment) return;  // not the expert's last block
        row = block0 + 1 + (pad_wave - b * p.pad_waves_per_expert);
    } else {
        e = (int)(pad_wave / p.pad_waves_per_expert);
        if (e >= p.num_experts) return;
        row = (int64_t)expert_psum[e] + expert_count[e] + (pad_wave - (int64_t)e * p.pad_waves_per_expert);
    }
    if (row < (int64_t)expert_psum[e] + expert_count[e] || row >= expert_psum[e + 1] || row >= p.recv_capacity)
        return;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const RowWriter dst(recv_x + row * p.row_vecs, (int)(p.row_vecs * 16));
    const int64_t v0 = (int64_t)part * p.pad_part_vecs;
    const int64_t v1 = min(p.row_vecs, v0 + p.pad_part_vecs);
    for (int64_t i = v0 + lane; i < v1; i += kWave) dst.store(i, zero);
    if (part != 0) return;  // the first part's wavefront zeroes the scale factors
    const int S = p.sf_per_token;
    for (int i = lane; i < S; i += kWave) recv_sf[row * S + i] = 0u;
}

template <int V, int W>
__global__ void __launch_bounds__(W * kWave)
scatter_kernel(const u32x4* __restrict__ x, const uint32_t* __restrict__ x_sf, ScatterParams p,
               const int32_t* __restrict__ expert_slot, const int32_t* __restrict__ rank_slot,
               const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_psum,
               const int32_t* __restrict__ status, u32x4* __restrict__ rank_x,
               uint32_t* __restrict__ rank_sf, u32x4* __restrict__ recv_x, uint32_t* __restrict__ recv_sf) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave_id = (int64_t)blockIdx.x * W + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (wave_id < p.token_waves) {
        const int64_t t = wave_id / p.segments;
        const int seg = (int)(wave_id - t * p.segments);
        if (t < p.num_tokens)
            copy_token<V>(x, x_sf, p, t, seg, lane, expert_slot, rank_slot, rank_x, rank_sf, recv_x, recv_sf,
                          status);
    } else {
        if (*status != 0) return;  // the layout is unspecified: write nothing
        zero_pads(p, wave_id - p.token_waves, lane, expert_count, expert_psum, recv_x, recv_sf);
    }
}

// Rows with many destinations (a dispatch: K expert rows and up to K rank
// rows per token) that the layout has just read into the Infinity Cache: one
// workgroup per (token, 1 KB row segment), whose wavefronts split the token's
// destinations, kSplitDestinations each. Every wavefront loads the segment
// itself (the workgroup's wavefronts share the CU's L1), issued with the
// status and slot loads so that one memory latency precedes the stores. The
// launch bounds how many workgroups share a CU (kSplitStoresPerCu): on MI355X
// the write stream ran faster with fewer row stores in flight, down to a
// cliff. Measured on the 4096 x 7168 bf16 batch (top-8 of 256 experts, 8
// ranks; 4 wavefronts per workgroup): 144 us at full occupancy, 134 / 129 /
// 153 / 213 us at 5 / 4 / 3 / 2 workgroups per CU; scatter_kernel, one
// wavefront per segment writing all its destinations, 143 us. With rows from
// HBM the bound slows it (163 against 216 us on the same batch) and the split
// itself loses (65 536 fp8 tokens: 1334 against 1198 us for scatter_kernel),
// so rows that were not read ahead take scatter_kernel. Pad rows follow as
// extra workgroups, 4 KB of a row per wavefront, about as many stores as a
// token wavefront issues (a whole 7 KB row per wavefront: 1 % slower on the
// 7 KB fp8 batch at alignment 128; 1 or 2 KB: 36 % and 14 % slower).
constexpr int kSplitDestinations = 4;
constexpr int kSplitStoresPerCu = 64;
constexpr int64_t kSplitPadVecs = 4 * kWave;  // a pad wavefront's vectors: 4 KB
constexpr int kWaveSlotsPerCu = 32;
constexpr int kMaxBoundedWorkgroupsPerCu = 8;

__global__ void __launch_bounds__(1024)
split_scatter_kernel(const u32x4* __restrict__ x, const uint32_t* __restrict__ x_sf, ScatterParams p,
                     const int32_t* __restrict__ expert_slot, const int32_t* __restrict__ rank_slot,
                     const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_psum,
                     const int32_t* __restrict__ status, u32x4* __restrict__ rank_x,
                     uint32_t* __restrict__ rank_sf, u32x4* __restrict__ recv_x, uint32_t* __restrict__ recv_sf) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int waves = blockDim.x / kWave;
    if ((int64_t)blockIdx.x >= p.token_groups) {  // pad rows, 4 KB per wavefront
        if (*status != 0) return;  // the layout is unspecified: write nothing
        zero_pads(p, ((int64_t)blockIdx.x - p.token_groups) * waves + wave, lane, expert_count, expert_psum, recv_x,
                  recv_sf);
        return;
    }
    const int K = p.num_topk;
    const int64_t t = blockIdx.x / p.segments;
    const int seg = (int)(blockIdx.x - t * p.segments);
    const int64_t nv = p.row_vecs;
    const int64_t i = (int64_t)seg * kWave + lane;
    const int S = seg == 0 ? p.sf_per_token : 0;  // the first segment's workgroup moves the scale factors
    // The segment, the status (a vector load, so that no wait for it holds
    // back the others) and the token's destinations: lanes [0, K) its expert
    // rows, lanes [K, 2K) its rank rows (at the owning k, else -1).
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i < nv) v = x[t * nv + i];
    uint32_t sf = 0;
    if (lane < S) sf = x_sf[t * S + lane];
    const int st = (int)__builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(status), 0, 4, kBufferWord3), 0, 0, 0);
    // One load instruction for both lists (a per-lane address, not two
    // branches, whose loads the compiler would serialize).
    const bool expert_lane = lane < K;
    const bool want = expert_lane ? p.write_expert != 0 : (lane < 2 * K && rank_slot != nullptr && p.write_rank != 0);
    const int32_t* slots = expert_lane ? expert_slot : rank_slot;
    int d = -1;
    if (want) d = slots[t * K + (expert_lane ? lane : lane - K)];
    asm volatile("" ::: "memory");  // the loads go out before the check below
    if (__builtin_amdgcn_readfirstlane(st) != 0) return;  // the layout is unspecified: write nothing
    // Slots past the capacities never occur with status 0; they are dropped
    // so that no store can leave the output buffers.
    if (expert_lane ? d >= p.recv_capacity : d >= p.rank_capacity) d = -1;
    uint64_t mine = __ballot(d >= 0);
    // This wavefront's destinations: the valid ones numbered
    // [wave * kSplitDestinations, (wave + 1) * kSplitDestinations).
    for (int skip = wave * kSplitDestinations; skip > 0 && mine != 0; --skip) mine &= mine - 1;
    for (int n = 0; n < kSplitDestinations && mine != 0; ++n, mine &= mine - 1) {
        const int j = __builtin_ctzll(mine);
        const int dest = __builtin_amdgcn_readlane(d, j);
        // Vectors past the row end fall outside the row's buffer range and are dropped.
        u32x4* row = (j < K ? recv_x : rank_x) + (int64_t)dest * nv;
        RowWriter(row, (int)(nv * 16)).store(i, v);
        if (S > 0) {
            uint32_t* sf_row = (j < K ? recv_sf : rank_sf) + (int64_t)dest * S;
            for (int q = lane; q < S; q += kWave) sf_row[q] = q < kWave ? sf : x_sf[t * S + q];
        }
    }
}

template <int V, int W>
hipError_t launch_v(dim3 grid, size_t lds, hipStream_t stream, const u32x4* x, const uint32_t* x_sf, ScatterParams p,
                    const int32_t* expert_slot, const int32_t* rank_slot, const int32_t* expert_count,
                    const int32_t* expert_psum, const int32_t* status, u32x4* rank_x, uint32_t* rank_sf,
                    u32x4* recv_x, uint32_t* recv_sf) {
    void* args[] = {&x, &x_sf, &p, &expert_slot, &rank_slot, &expert_count, &expert_psum,
                    &status, &rank_x, &rank_sf, &recv_x, &recv_sf};
    return hipLaunchKernel(reinterpret_cast<const void*>(&scatter_kernel<V, W>), grid, dim3(W * kWave), args, lds,
                           stream);
}

// The scatter's parameters and grid for a problem: workgroups and threads
// per workgroup, the token workgroups first, then the pad-row wavefronts.
struct ScatterLaunch {
    ScatterParams p;
    bool split;        // split_scatter_kernel, else scatter_kernel
    int v;             // 16-byte vectors per lane of scatter_kernel
    int64_t blocks;
    int threads;
    int lds;           // dynamic LDS per workgroup, reserved only to bound the workgroups per CU
};

ScatterLaunch plan_scatter(const dispatch_problem_t& prob, bool few_destinations) {
    ScatterLaunch s{};
    ScatterParams& p = s.p;
    p.num_tokens = prob.num_tokens;
    p.row_vecs = prob.row_bytes / 16;
    // Segments of about max_vecs vectors per lane, balanced over the row.
    const int max_vecs = few_destinations ? kVecsFewDestinations : kVecsManyDestinations;
    p.segments = (int32_t)((p.row_vecs + kWave * max_vecs - 1) / (kWave * max_vecs));
    if (p.segments < 1) p.segments = 1;
    const int64_t seg_vecs = (p.row_vecs + p.segments - 1) / p.segments;
    s.v = (int)((seg_vecs + kWave - 1) / kWave);
    // A token's destinations at most: K expert rows and min(K, R) rank rows.
    const int list = ((prob.flags & DISPATCH_EXPERT_MAJOR) ? prob.num_topk : 0) +
                     ((prob.flags & DISPATCH_RANK_CONTIG) ? (prob.num_topk < prob.num_ranks ? prob.num_topk
                                                                                              : prob.num_ranks)
                                                          : 0);
    // Rows read ahead into the Infinity Cache (the hint, and rows that
    // dispatch_layout_read_ahead does read) take the split kernel.
    const bool cached = (prob.flags & DISPATCH_ROWS_READ_AHEAD) &&
                        read_ahead_fits(prob.num_tokens * prob.row_bytes, prob.num_tokens * prob.sf_per_token);
    s.split = !few_destinations && cached;
    const int split_waves = list < 1 ? 1 : (list + kSplitDestinations - 1) / kSplitDestinations;
    const int w = s.split ? split_waves : (few_destinations ? kWavesFewDestinations : kWavesManyDestinations);
    s.threads = w * kWave;
    const int64_t waves = prob.num_tokens * p.segments;
    p.token_waves = (waves + w - 1) / w * w;
    p.recv_capacity = prob.recv_capacity_rows;
    p.rank_capacity = prob.rank_capacity_rows;
    p.num_topk = prob.num_topk;
    p.sf_per_token = prob.sf_per_token;
    p.num_experts = prob.num_experts;
    p.write_rank = (prob.flags & DISPATCH_RANK_CONTIG) != 0;
    p.write_expert = (prob.flags & DISPATCH_EXPERT_MAJOR) != 0;
    const bool pads = p.write_expert && (prob.flags & DISPATCH_ZERO_PAD) && prob.expert_alignment > 1;
    p.alignment = prob.expert_alignment;
    p.pad_waves_per_expert = pads ? prob.expert_alignment - 1 : 1;
    // Blocks of `alignment` receive rows that routed rows can reach: each
    // routed expert ends in one partly filled block, the rest are full.
    const int64_t pairs = prob.num_tokens * prob.num_topk;
    const int64_t blocks_reached = (pairs < prob.num_experts ? pairs : prob.num_experts) +
                                   pairs / prob.expert_alignment;
    p.pad_by_block = blocks_reached < prob.num_experts;
    // The split kernel's pad wavefronts zero at most kSplitPadVecs vectors
    // each, about as many stores as its token wavefronts issue; the other
    // kernel's zero whole rows.
    p.pad_part_vecs = s.split ? kSplitPadVecs : (p.row_vecs > 0 ? p.row_vecs : 1);
    p.pad_parts = p.row_vecs > p.pad_part_vecs ? (int32_t)((p.row_vecs + p.pad_part_vecs - 1) / p.pad_part_vecs) : 1;
    const int64_t pad_waves =
        pads ? (p.pad_by_block ? blocks_reached : (int64_t)prob.num_experts) * p.pad_waves_per_expert * p.pad_parts
             : 0;
    p.token_groups = prob.num_tokens * p.segments;
    if (s.split) {
        s.blocks = p.token_groups + (pad_waves + w - 1) / w;
        // About kSplitStoresPerCu row stores in flight per CU, each
        // workgroup issuing up to `list`. The bound was measured with 1 to 8
        // workgroups per CU (8 to 64 destinations per token); fewer
        // destinations per token, and bounds a CU's wavefront slots impose
        // anyway, run unbounded.
        const int per_cu = (kSplitStoresPerCu + list - 1) / (list < 1 ? 1 : list);
        s.lds = per_cu <= kMaxBoundedWorkgroupsPerCu && per_cu * w < kWaveSlotsPerCu
                    ? lds_for_workgroups_per_cu(per_cu)
                    : 0;
    } else {
        s.blocks = (p.token_waves + pad_waves + w - 1) / w;
    }
    return s;
}

}  // namespace

bool scatter_grid_fits(const dispatch_problem_t& prob, bool few_destinations) {
    const ScatterLaunch s = plan_scatter(prob, few_destinations);
    // One grid dimension: at most 2^31 - 1 workgroups and 2^32 - 1 work-items.
    return s.blocks <= INT32_MAX && s.blocks * s.threads <= (int64_t)UINT32_MAX;
}

hipError_t launch_scatter(const dispatch_problem_t& prob, const dispatch_layout_t& lay, const void* x,
                          const float* x_sf, void* rank_x, float* rank_sf, void* recv_x, float* recv_sf,
                          hipStream_t stream, bool few_destinations) {
    const ScatterLaunch s = plan_scatter(prob, few_destinations);
    if (s.blocks == 0) return hipSuccess;
    if (s.blocks > INT32_MAX || s.blocks * s.threads > (int64_t)UINT32_MAX)
        return hipErrorInvalidConfiguration;  // beyond one grid: refused, never truncated
    const dim3 grid((unsigned)s.blocks);
    const size_t lds = (size_t)s.lds;
    const ScatterParams& p = s.p;
    auto* xs = static_cast<const u32x4*>(x);
    auto* sfs = reinterpret_cast<const uint32_t*>(x_sf);
    auto* rx = static_cast<u32x4*>(rank_x);
    auto* rsf = reinterpret_cast<uint32_t*>(rank_sf);
    auto* ex = static_cast<u32x4*>(recv_x);
    auto* esf = reinterpret_cast<uint32_t*>(recv_sf);
    if (s.split) {
        const int32_t* es = lay.expert_slot;
        const int32_t* rs = lay.rank_slot;
        const int32_t* ec = lay.expert_count;
        const int32_t* ep = lay.expert_psum;
        const int32_t* st = lay.status;
        ScatterParams pc = p;
        void* args[] = {&xs, &sfs, &pc, &es, &rs, &ec, &ep, &st, &rx, &rsf, &ex, &esf};
        return hipLaunchKernel(reinterpret_cast<const void*>(&split_scatter_kernel), grid, dim3(s.threads), args, lds,
                               stream);
    }
#define MOE_DISPATCH_SCATTER_CASE(N)                                                                       \
    case N:                                                                                                \
        return launch_v<N, kWavesFewDestinations>(grid, lds, stream, xs, sfs, p, lay.expert_slot, lay.rank_slot, \
                                                  lay.expert_count, lay.expert_psum, lay.status, rx, rsf, ex, esf);
    if (!few_destinations)  // one vector per lane (kVecsManyDestinations)
        return launch_v<kVecsManyDestinations, kWavesManyDestinations>(grid, lds, stream, xs, sfs, p, lay.expert_slot,
                                                                       lay.rank_slot, lay.expert_count,
                                                                       lay.expert_psum, lay.status, rx, rsf, ex, esf);
    switch (s.v) {
        MOE_DISPATCH_SCATTER_CASE(1)
        MOE_DISPATCH_SCATTER_CASE(2)
        MOE_DISPATCH_SCATTER_CASE(3)
        default:
            return launch_v<4, kWavesFewDestinations>(grid, lds, stream, xs, sfs, p, lay.expert_slot, lay.rank_slot,
                                                      lay.expert_count, lay.expert_psum, lay.status, rx, rsf, ex, esf);
    }
#undef MOE_DISPATCH_SCATTER_CASE
}

}  // namespace moe_dispatch
