// Row scatter on gfx950: copy each token row into its rank-contiguous rows and
// its expert-major rows, and zero the alignment pad rows.
//
// This is the data move of the method ("DeepEP Counting Sort / Bucketization"
// page): the rank-level copy of sections 6.2-6.3, the expert-major copy of the
// expand mode (sections 6.4 and 8.2) and the zero padding of section 7.3. It
// moves nearly all of the bytes, so it is built for HBM bandwidth: a token
// row is cut into segments of 64 x V 16-byte vectors, and one wavefront per
// (token, segment) reads its segment once, 16 bytes per lane per instruction,
// holds it in registers and writes it to every destination row of that token
// (the read-once / write-to-many-destinations copy of the "Symmetric Memory"
// page's sender warp, here to local rows). Destination slots come from the
// layout's expert_slot / rank_slot, which are wavefront-uniform, so the
// destination loop runs on scalar registers. Pad rows are cleared by extra
// wavefronts after the token wavefronts, one row each.
//
// Row stores go through a buffer resource that spans exactly one destination
// row, so the hardware drops any offset outside that row, and carry the
// streaming cache policy (nt with sc1): the output is far larger than the
// caches and is not read back here, and of the store forms measured on MI355X
// this one moved the rows fastest.
#include "dispatch_common.hpp"
#include "dispatch_device.hpp"

namespace moe_dispatch {
namespace {

static_assert(DISPATCH_MAX_EXPERTS <= kWave * kWave, "expert_of_row searches two rounds of 64 samples");
// V, the 16-byte vectors per lane of one row segment, follows the stores per
// loaded row (measured on MI355X): with many destinations per row (dispatch:
// K expert rows and the rank rows) one vector per lane, i.e. many short
// wavefronts, moves the rows fastest; with about one destination per row
// (the receiver-side expand, a top-1 copy) four vectors per lane do.
constexpr int kVecsManyDestinations = 1;
constexpr int kVecsFewDestinations = 4;
// Wavefronts per workgroup, measured the same way: 1 with many destinations
// per row, 4 with about one.
constexpr int kWavesManyDestinations = 1;
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
    int32_t pad_waves_per_expert;  // alignment - 1 with pads, else 1
    int32_t pad_by_block;          // pad wavefronts mapped per row block (else per expert)
    int32_t alignment;
    int32_t write_rank;      // rank_x / rank_sf requested
    int32_t write_expert;    // recv_x / recv_sf requested
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
    for (int64_t i = lane; i < p.row_vecs; i += kWave) dst.store(i, zero);
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

// Row scatter in destination order, for layouts that keep a row order
// (keeps_row_order: rows of 4 to 8 KB with several destinations each, read
// ahead into the Infinity Cache). The order lists every
// routed row as (dest, token), tile by tile (a tile is a run of consecutive
// tokens), inside a tile grouped by expert then rank, each group in slot
// order. Workgroup b takes kOrderWaves * kOrderRows consecutive entries and
// one slice (of about 3.5 KB) of their rows: b / slices picks the entries,
// b % slices the slice. Workgroups run on XCD b % 8, so each XCD's L2 holds
// only a slice of the current tile's source rows, and consecutive workgroups
// fill consecutive destination rows. Each destination row is written once;
// each source row is read once per destination, from the caches (the layout
// kernels read the rows ahead into the Infinity Cache). On MI355X this moved
// 7 KB fp8 rows with scale factors 5 % faster than one wavefront per source
// row segment writing all of its destinations (98 against 104 us for 4096
// tokens, top-8 of 256, alignment 128); 4 wavefronts of 2 rows and slices of
// at most 4 KB measured best.
constexpr int kOrderRows = 2;          // order entries (destination rows) per wavefront
constexpr int kOrderWaves = 4;         // wavefronts per workgroup
constexpr int kOrderSliceMaxVecs = 256;  // 16-byte vectors per row slice, at most (4 per lane)

struct OrderShape {
    int64_t groups;       // workgroups per slice (entries / (kOrderWaves * kOrderRows), rounded up)
    int64_t max_entries;  // entries the order can hold
    int32_t slices;
    int32_t slice_vecs;
};

inline OrderShape order_shape(const dispatch_problem_t& prob) {
    OrderShape o{};
    const int64_t row_vecs = prob.row_bytes / 16;
    o.slices = (int32_t)((row_vecs + kOrderSliceMaxVecs - 1) / kOrderSliceMaxVecs);
    o.slice_vecs = (int32_t)((row_vecs + o.slices - 1) / o.slices);
    o.max_entries = (row_order_ints(prob) - 2) / 2;
    o.groups = (o.max_entries + kOrderWaves * kOrderRows - 1) / (kOrderWaves * kOrderRows);
    return o;
}

template <int SV>
__global__ void __launch_bounds__(kOrderWaves * kWave)
order_scatter_kernel(const u32x4* __restrict__ x, const uint32_t* __restrict__ x_sf, ScatterParams p, OrderShape o,
                     const int2* __restrict__ order, const int32_t* __restrict__ expert_count,
                     const int32_t* __restrict__ expert_psum, const int32_t* __restrict__ status,
                     u32x4* __restrict__ rank_x, uint32_t* __restrict__ rank_sf, u32x4* __restrict__ recv_x,
                     uint32_t* __restrict__ recv_sf) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t order_blocks = o.groups * o.slices;
    if ((int64_t)blockIdx.x >= order_blocks) {  // pad rows, one per wavefront
        if (*status != 0) return;  // the layout is unspecified: write nothing
        zero_pads(p, ((int64_t)blockIdx.x - order_blocks) * kOrderWaves + wave, lane, expert_count, expert_psum,
                  recv_x, recv_sf);
        return;
    }
    const int64_t group = blockIdx.x / o.slices;
    const int j = (int)(blockIdx.x - group * o.slices);
    const int64_t first = (group * kOrderWaves + wave) * kOrderRows;
    // The status, the entry count and this wavefront's entries are loaded
    // together (entries past the count lie inside the array and are dropped
    // below), so that one memory latency, not three, precedes the row loads.
    const int st = *status;
    const int64_t count = order[0].x;
    int2 ent = make_int2(0, -1);
    if (lane < kOrderRows && first + lane < o.max_entries) ent = order[1 + first + lane];
    asm volatile("" ::: "memory");  // the three loads go out before the checks below
    if (st != 0) return;  // the layout is unspecified: write nothing
    const int64_t n = min(count, o.max_entries);
    if (first >= n) return;
    if (first + lane >= n) ent.y = -1;
    const int64_t nv = p.row_vecs;
    const int64_t v0 = (int64_t)j * o.slice_vecs;
    const int64_t v1 = min(v0 + o.slice_vecs, nv);
    // All loads of the wavefront's rows go out before the first store.
    u32x4 v[kOrderRows][SV];
    int src[kOrderRows];
#pragma unroll
    for (int r = 0; r < kOrderRows; ++r) {
        const int t = __builtin_amdgcn_readlane(ent.y, r);
        src[r] = t >= 0 && t < p.num_tokens ? t : -1;
#pragma unroll
        for (int q = 0; q < SV; ++q) {
            const int64_t i = v0 + q * kWave + lane;
            if (src[r] >= 0 && i < v1) v[r][q] = x[(int64_t)src[r] * nv + i];
        }
    }
#pragma unroll
    for (int r = 0; r < kOrderRows; ++r) {
        if (src[r] < 0) continue;
        const int d = __builtin_amdgcn_readlane(ent.x, r);
        u32x4* row;
        uint32_t* sf_row;
        if (d >= 0) {
            if (!p.write_expert || d >= p.recv_capacity) continue;
            row = recv_x + (int64_t)d * nv;
            sf_row = recv_sf + (int64_t)d * p.sf_per_token;
        } else {
            const int64_t rr = -1 - (int64_t)d;
            if (!p.write_rank || rr >= p.rank_capacity) continue;
            row = rank_x + rr * nv;
            sf_row = rank_sf + rr * p.sf_per_token;
        }
        const RowWriter dst(row, (int)(nv * 16));
#pragma unroll
        for (int q = 0; q < SV; ++q) {
            const int64_t i = v0 + q * kWave + lane;
            if (i < v1) dst.store(i, v[r][q]);
        }
        if (j == 0)  // the first slice's wavefronts move the scale factors
            for (int i = lane; i < p.sf_per_token; i += kWave)
                sf_row[i] = x_sf[(int64_t)src[r] * p.sf_per_token + i];
    }
}

template <int V, int W>
hipError_t launch_v(dim3 grid, hipStream_t stream, const u32x4* x, const uint32_t* x_sf, ScatterParams p,
                    const int32_t* expert_slot, const int32_t* rank_slot, const int32_t* expert_count,
                    const int32_t* expert_psum, const int32_t* status, u32x4* rank_x, uint32_t* rank_sf,
                    u32x4* recv_x, uint32_t* recv_sf) {
    void* args[] = {&x, &x_sf, &p, &expert_slot, &rank_slot, &expert_count, &expert_psum,
                    &status, &rank_x, &rank_sf, &recv_x, &recv_sf};
    return hipLaunchKernel(reinterpret_cast<const void*>(&scatter_kernel<V, W>), grid, dim3(W * kWave), args, 0,
                           stream);
}

template <int SV>
hipError_t launch_order_sv(dim3 grid, hipStream_t stream, const u32x4* x, const uint32_t* x_sf, ScatterParams p,
                           OrderShape o, const int2* order, const int32_t* expert_count, const int32_t* expert_psum,
                           const int32_t* status, u32x4* rank_x, uint32_t* rank_sf, u32x4* recv_x,
                           uint32_t* recv_sf) {
    void* args[] = {&x, &x_sf, &p, &o, &order, &expert_count, &expert_psum, &status, &rank_x, &rank_sf, &recv_x,
                    &recv_sf};
    return hipLaunchKernel(reinterpret_cast<const void*>(&order_scatter_kernel<SV>), grid, dim3(kOrderWaves * kWave),
                           args, 0, stream);
}

// Whether a scatter of this problem takes the ordered kernel.
inline bool takes_order(const dispatch_problem_t& prob, const dispatch_layout_t& lay, bool few_destinations) {
    return lay.row_order != nullptr && !few_destinations && keeps_row_order(prob);
}

// The scatter's parameters and grid for a problem: workgroups and threads
// per workgroup, token wavefronts first (or the ordered kernel's entry
// groups), then the pad-row wavefronts.
struct ScatterLaunch {
    ScatterParams p;
    bool order;
    OrderShape o;
    int v;             // 16-byte vectors per lane of the source-major kernel
    int64_t blocks;
    int threads;
};

ScatterLaunch plan_scatter(const dispatch_problem_t& prob, const dispatch_layout_t& lay, bool few_destinations) {
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
    s.order = takes_order(prob, lay, few_destinations);
    const int w = s.order ? kOrderWaves : (few_destinations ? kWavesFewDestinations : kWavesManyDestinations);
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
    const int64_t pad_waves =
        pads ? (p.pad_by_block ? blocks_reached : (int64_t)prob.num_experts) * p.pad_waves_per_expert : 0;
    if (s.order) {
        s.o = order_shape(prob);
        s.blocks = s.o.groups * s.o.slices + (pad_waves + w - 1) / w;
    } else {
        s.blocks = (p.token_waves + pad_waves + w - 1) / w;
    }
    return s;
}

}  // namespace

bool scatter_grid_fits(const dispatch_problem_t& prob, const dispatch_layout_t& lay, bool few_destinations) {
    const ScatterLaunch s = plan_scatter(prob, lay, few_destinations);
    // One grid dimension: at most 2^31 - 1 workgroups and 2^32 - 1 work-items.
    return s.blocks <= INT32_MAX && s.blocks * s.threads <= (int64_t)UINT32_MAX;
}

hipError_t launch_scatter(const dispatch_problem_t& prob, const dispatch_layout_t& lay, const void* x,
                          const float* x_sf, void* rank_x, float* rank_sf, void* recv_x, float* recv_sf,
                          hipStream_t stream, bool few_destinations) {
    const ScatterLaunch s = plan_scatter(prob, lay, few_destinations);
    if (s.blocks == 0) return hipSuccess;
    if (s.blocks > INT32_MAX || s.blocks * s.threads > (int64_t)UINT32_MAX)
        return hipErrorInvalidConfiguration;  // beyond one grid: refused, never truncated
    const dim3 grid((unsigned)s.blocks);
    const ScatterParams& p = s.p;
    auto* xs = static_cast<const u32x4*>(x);
    auto* sfs = reinterpret_cast<const uint32_t*>(x_sf);
    auto* rx = static_cast<u32x4*>(rank_x);
    auto* rsf = reinterpret_cast<uint32_t*>(rank_sf);
    auto* ex = static_cast<u32x4*>(recv_x);
    auto* esf = reinterpret_cast<uint32_t*>(recv_sf);
    if (s.order) {
        const auto* order = reinterpret_cast<const int2*>(lay.row_order);
        switch ((s.o.slice_vecs + kWave - 1) / kWave) {
            case 1: return launch_order_sv<1>(grid, stream, xs, sfs, p, s.o, order, lay.expert_count,
                                              lay.expert_psum, lay.status, rx, rsf, ex, esf);
            case 2: return launch_order_sv<2>(grid, stream, xs, sfs, p, s.o, order, lay.expert_count,
                                              lay.expert_psum, lay.status, rx, rsf, ex, esf);
            case 3: return launch_order_sv<3>(grid, stream, xs, sfs, p, s.o, order, lay.expert_count,
                                              lay.expert_psum, lay.status, rx, rsf, ex, esf);
            default: return launch_order_sv<4>(grid, stream, xs, sfs, p, s.o, order, lay.expert_count,
                                               lay.expert_psum, lay.status, rx, rsf, ex, esf);
        }
    }
    if (!few_destinations)  // one vector per lane: v == 1
        return launch_v<1, kWavesManyDestinations>(grid, stream, xs, sfs, p, lay.expert_slot, lay.rank_slot,
                                                   lay.expert_count, lay.expert_psum, lay.status, rx, rsf, ex, esf);
#define MOE_DISPATCH_SCATTER_CASE(N)                                                                       \
    case N:                                                                                                \
        return launch_v<N, kWavesFewDestinations>(grid, stream, xs, sfs, p, lay.expert_slot, lay.rank_slot, \
                                                  lay.expert_count, lay.expert_psum, lay.status, rx, rsf, ex, esf);
    switch (s.v) {
        MOE_DISPATCH_SCATTER_CASE(1)
        MOE_DISPATCH_SCATTER_CASE(2)
        MOE_DISPATCH_SCATTER_CASE(3)
        default:
            return launch_v<4, kWavesFewDestinations>(grid, stream, xs, sfs, p, lay.expert_slot, lay.rank_slot,
                                                      lay.expert_count, lay.expert_psum, lay.status, rx, rsf, ex, esf);
    }
#undef MOE_DISPATCH_SCATTER_CASE
}

}  // namespace moe_dispatch
