// Dispatch layout on gfx950: Count -> Prefix Sum -> stable slot assignment.
//
// The method ("DeepEP Counting Sort / Bucketization" page) counts the routed
// (token, expert) pairs per expert and the distinct (token, rank) pairs per
// rank (section 4.2), takes exclusive prefix sums over the expert counts
// aligned up to the expert alignment and over the rank counts (sections 5.2
// and 7.2), and gives every pair a slot inside its bucket (sections 6.2 and
// 6.4). The page's kernel lets shared-memory and global atomics decide the
// order inside a bucket; here the order is ascending token index, and no
// atomic decides a slot.
//
// Two kernels, both one workgroup per tile of consecutive tokens:
//
//   count_kernel   Each wavefront ranks its sub-tile's pairs chunk by chunk
//                  (see rank_chunk) into wavefront-private LDS counters, the
//                  workgroup adds them into a tile histogram, and the last
//                  workgroup to finish (a ticket counter; nobody waits on
//                  anybody) turns all tile histograms into the counts, the
//                  aligned exclusive psums and, per tile, the base slot of
//                  every key. It then clears the ticket so the workspace is
//                  ready for the next call without a memset.
//   assign_kernel  Each tile ranks its pairs again the same way, scans the
//                  wavefront counters into sub-tile bases on top of the tile
//                  base, and writes expert_slot, rank_slot and the inverse
//                  maps; pad entries of recv_src_token_idx become -1.
//
// Rank dedup: among the lanes of one token, the pair that owns a rank is the
// highest k in that rank (the page's "master lane"). gfx950 has no match-any
// instruction, so lanes holding equal keys are found with one ballot per key
// bit (a wavefront multisplit).
#include "dispatch_common.hpp"

namespace moe_dispatch {
namespace {

struct LayoutParams {
    int64_t num_tokens;
    int64_t recv_capacity;
    int64_t rank_capacity;
    int32_t num_topk;
    int32_t num_experts;
    int32_t num_ranks;
    int32_t experts_per_rank;
    int32_t alignment;
    int32_t expert_bits;  // bits needed for an expert id
    int32_t rank_bits;    // bits needed for a rank id
    int32_t tokens_per_chunk;
    int32_t tokens_per_wave;
    int32_t tokens_per_tile;
    int32_t num_keys;
    int32_t num_tiles;
};

// Where one lane's pair lands inside its wavefront's sub-tile.
struct PairPos {
    int expert;      // expert id, or -1 when the lane holds no routed pair
    int expert_pos;  // earlier pairs of that expert in the sub-tile
    int rank;        // rank id when the lane owns its (token, rank), else -1
    int rank_pos;    // earlier owned (token, rank) pairs of that rank in the sub-tile
};

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }
__device__ __forceinline__ uint64_t lanes_above(int lane) {
    return lane == kWave - 1 ? 0ull : (~0ull << (lane + 1));
}

// Lanes whose key equals this lane's key: one ballot per key bit.
__device__ __forceinline__ uint64_t match_key(int key, int bits) {
    uint64_t same = ~0ull;
    for (int b = 0; b < bits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t set = __ballot(bit);
        same &= bit ? set : ~set;
    }
    return same;
}

__device__ __forceinline__ void wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Rank one chunk of pairs. `entry` is this lane's topk entry (-1 for lanes
// beyond the chunk or the tile). `counters` holds the wavefront's running
// count of every key over the chunks already ranked; it is advanced by this
// chunk. Must be called by all 64 lanes together.
__device__ __forceinline__ PairPos rank_chunk(int64_t entry, int lane, int token_in_chunk,
                                              const LayoutParams& p, int* __restrict__ counters,
                                              uint32_t& err) {
    const int K = p.num_topk;
    const bool bad = entry >= p.num_experts;
    const bool valid = entry >= 0 && !bad;
    const int e = valid ? (int)entry : 0;
    const int r = e / p.experts_per_rank;

    const uint64_t routed = __ballot(valid);
    const uint64_t same_expert = routed & match_key(e, p.expert_bits);
    const uint64_t same_rank = routed & match_key(r, p.rank_bits);
    const uint64_t own_token = (((K == 64) ? ~0ull : ((1ull << K) - 1ull))) << (token_in_chunk * K);
    const uint64_t below = lanes_below(lane), above = lanes_above(lane);

    if (valid && __popcll(same_expert & own_token) > 1) err |= DISPATCH_STATUS_DUP_EXPERT;
    if (bad) err |= DISPATCH_STATUS_BAD_EXPERT;

    // The highest k of a rank inside the token owns the (token, rank) pair.
    const bool owner = valid && (same_rank & own_token & above) == 0ull;
    const uint64_t same_rank_owner = same_rank & __ballot(owner);

    const int e_before = __popcll(same_expert & below);
    const int r_before = __popcll(same_rank_owner & below);
    const int e_base = valid ? counters[e] : 0;
    const int r_base = owner ? counters[p.num_experts + r] : 0;
    wave_fence();
    // The highest lane of every key group advances that key's counter.
    if (valid && (same_expert & above) == 0ull) counters[e] = e_base + e_before + 1;
    if (owner && (same_rank_owner & above) == 0ull) counters[p.num_experts + r] = r_base + r_before + 1;
    wave_fence();

    PairPos pos;
    pos.expert = valid ? e : -1;
    pos.expert_pos = e_base + e_before;
    pos.rank = owner ? r : -1;
    pos.rank_pos = r_base + r_before;
    return pos;
}

template <typename IdxT>
__device__ __forceinline__ void load_entries(const IdxT* __restrict__ topk, int64_t wave_tok0,
                                             int64_t tile_end, int lane, int token_in_chunk, int k,
                                             const LayoutParams& p, int64_t (&entry)[kChunksPerWave]) {
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
        const int64_t tok = wave_tok0 + (int64_t)c * p.tokens_per_chunk + token_in_chunk;
        const bool live = token_in_chunk < p.tokens_per_chunk && tok < tile_end;
        entry[c] = live ? (int64_t)topk[tok * p.num_topk + k] : -1;
    }
}

// Exclusive scan, in place, of up to n LDS values (each rounded up to a
// multiple of `align` first) by the whole workgroup. Returns the total.
__device__ int block_exclusive_scan(int* __restrict__ v, int n, int align, int* __restrict__ scratch) {
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = nthreads / kWave;
    const int per = (n + nthreads - 1) / nthreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int local = 0;
    for (int i = lo; i < hi; ++i) {
        const int c = v[i];
        local += align > 1 ? (c + align - 1) / align * align : c;
    }
    // Kogge-Stone inclusive scan across the 64 lanes (6 steps).
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int up = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += up;
    }
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < nwaves; ++w) {
            const int t = scratch[w];
            scratch[w] = run;
            run += t;
        }
        scratch[nwaves] = run;
    }
    __syncthreads();
    int run = scratch[wave] + incl - local;
    for (int i = lo; i < hi; ++i) {
        const int c = v[i];
        v[i] = run;
        run += align > 1 ? (c + align - 1) / align * align : c;
    }
    const int total = scratch[nwaves];
    __syncthreads();
    return total;
}

template <typename IdxT>
__global__ void __launch_bounds__(1024)
count_kernel(const IdxT* __restrict__ topk, LayoutParams p, WorkspaceHeader* __restrict__ hdr,
             int32_t* __restrict__ tile_hist, int32_t* __restrict__ tile_base, dispatch_layout_t out) {
    extern __shared__ int lds[];  // [W][num_keys] wavefront counters
    __shared__ int scratch[kMaxWavesPerTile + 1];
    __shared__ uint32_t block_err;
    __shared__ int is_last;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nthreads = blockDim.x, nwaves = nthreads / kWave, nkeys = p.num_keys;
    int* counters = lds + wave * nkeys;
    for (int i = lane; i < nkeys; i += kWave) counters[i] = 0;
    if (tid == 0) block_err = 0;
    __syncthreads();

    const int token_in_chunk = lane / p.num_topk;
    const int k = lane - token_in_chunk * p.num_topk;
    const int64_t tile_tok0 = (int64_t)blockIdx.x * p.tokens_per_tile;
    const int64_t tile_end = min(p.num_tokens, tile_tok0 + p.tokens_per_tile);
    const int64_t wave_tok0 = tile_tok0 + (int64_t)wave * p.tokens_per_wave;

    int64_t entry[kChunksPerWave];
    load_entries(topk, wave_tok0, tile_end, lane, token_in_chunk, k, p, entry);
    uint32_t err = 0;
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) (void)rank_chunk(entry[c], lane, token_in_chunk, p, counters, err);
    const uint64_t any_bad = __ballot((err & DISPATCH_STATUS_BAD_EXPERT) != 0);
    const uint64_t any_dup = __ballot((err & DISPATCH_STATUS_DUP_EXPERT) != 0);
    if (lane == 0 && (any_bad | any_dup))
        atomicOr(&block_err, (any_bad ? DISPATCH_STATUS_BAD_EXPERT : 0u) | (any_dup ? DISPATCH_STATUS_DUP_EXPERT : 0u));
    __syncthreads();

    // Tile histogram: sum of the wavefront counters.
    int32_t* my_hist = tile_hist + (int64_t)blockIdx.x * nkeys;
    for (int j = tid; j < nkeys; j += nthreads) {
        int s = 0;
        for (int w = 0; w < nwaves; ++w) s += lds[w * nkeys + j];
        my_hist[j] = s;
    }
    if (tid == 0 && block_err)
        __hip_atomic_fetch_or(&hdr->error_bits, block_err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Release this tile's histogram device-wide, then take a ticket.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t ticket =
            __hip_atomic_fetch_add(&hdr->ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        is_last = ticket == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();  // acquire every other tile's histogram

    // ---- Last workgroup: counts, psums and per-tile key bases. ----
    const int E = p.num_experts, R = p.num_ranks;
    int* totals = lds;  // the wavefront counters are no longer needed
    for (int j = tid; j < nkeys; j += nthreads) {
        int s = 0;
        for (int i = 0; i < p.num_tiles; ++i) s += tile_hist[(int64_t)i * nkeys + j];
        totals[j] = s;
    }
    __syncthreads();
    for (int j = tid; j < nkeys; j += nthreads) {
        if (j < E) out.expert_count[j] = totals[j];
        else out.rank_count[j - E] = totals[j];
    }
    __syncthreads();
    // Exclusive psums (alignment before the sum, section 7.2); totals[] now
    // holds each key's first slot.
    const int recv_rows = block_exclusive_scan(totals, E, p.alignment, scratch);
    const int rank_rows = block_exclusive_scan(totals + E, R, 1, scratch);
    for (int j = tid; j < nkeys; j += nthreads) {
        if (j < E) out.expert_psum[j] = totals[j];
        else out.rank_psum[j - E] = totals[j];
    }
    // Per-tile base slot of every key: the key's first slot plus the pairs
    // of that key in earlier tiles.
    for (int j = tid; j < nkeys; j += nthreads) {
        int run = totals[j];
        for (int i = 0; i < p.num_tiles; ++i) {
            const int h = tile_hist[(int64_t)i * nkeys + j];
            tile_base[(int64_t)i * nkeys + j] = run;
            run += h;
        }
    }
    if (tid == 0) {
        out.expert_psum[E] = recv_rows;
        out.rank_psum[R] = rank_rows;
        uint32_t status = __hip_atomic_load(&hdr->error_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (recv_rows > p.recv_capacity) status |= DISPATCH_STATUS_RECV_OVERFLOW;
        if (rank_rows > p.rank_capacity) status |= DISPATCH_STATUS_RANK_OVERFLOW;
        *out.status = (int32_t)status;
        // Leave the control words zero for the next call.
        __hip_atomic_store(&hdr->error_bits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&hdr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <typename IdxT>
__global__ void __launch_bounds__(1024)
assign_kernel(const IdxT* __restrict__ topk, LayoutParams p, const int32_t* __restrict__ tile_base,
              dispatch_layout_t out) {
    if (*out.status != 0) return;  // the layout is unspecified: write nothing
    extern __shared__ int lds[];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nthreads = blockDim.x, nwaves = nthreads / kWave, nkeys = p.num_keys;
    const int K = p.num_topk, E = p.num_experts;
    int* counters = lds + wave * nkeys;
    for (int i = lane; i < nkeys; i += kWave) counters[i] = 0;
    wave_fence();

    const int token_in_chunk = lane / K;
    const int k = lane - token_in_chunk * K;
    const int64_t tile_tok0 = (int64_t)blockIdx.x * p.tokens_per_tile;
    const int64_t tile_end = min(p.num_tokens, tile_tok0 + p.tokens_per_tile);
    const int64_t wave_tok0 = tile_tok0 + (int64_t)wave * p.tokens_per_wave;

    int64_t entry[kChunksPerWave];
    load_entries(topk, wave_tok0, tile_end, lane, token_in_chunk, k, p, entry);
    uint32_t err = 0;
    PairPos pos[kChunksPerWave];
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) pos[c] = rank_chunk(entry[c], lane, token_in_chunk, p, counters, err);
    __syncthreads();

    // Sub-tile bases: scan the wavefront counters of each key in wavefront
    // order, on top of the tile's base slot for that key.
    const int32_t* my_base = tile_base + (int64_t)blockIdx.x * nkeys;
    for (int j = tid; j < nkeys; j += nthreads) {
        int run = my_base[j];
        for (int w = 0; w < nwaves; ++w) {
            const int c = lds[w * nkeys + j];
            lds[w * nkeys + j] = run;
            run += c;
        }
    }
    __syncthreads();

#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
        const int64_t tok = wave_tok0 + (int64_t)c * p.tokens_per_chunk + token_in_chunk;
        const bool live = token_in_chunk < p.tokens_per_chunk && tok < tile_end;
        if (!live) continue;
        const int es = pos[c].expert >= 0 ? counters[pos[c].expert] + pos[c].expert_pos : -1;
        const int rs = pos[c].rank >= 0 ? counters[E + pos[c].rank] + pos[c].rank_pos : -1;
        out.expert_slot[tok * K + k] = es;
        out.rank_slot[tok * K + k] = rs;
        // Slots are below the totals, which fit the capacities when the
        // status is 0; the bounds are checked anyway before every store.
        if (es >= 0 && es < p.recv_capacity) out.recv_src_token_idx[es] = (int32_t)tok;
        if (rs >= 0 && rs < p.rank_capacity) out.rank_src_token_idx[rs] = (int32_t)tok;
    }

    // Alignment pads of recv_src_token_idx (section 7.3): the slots after an
    // expert's real rows up to its aligned end map to no token.
    if (p.alignment > 1) {
        for (int e = blockIdx.x; e < E; e += gridDim.x) {
            const int lo = out.expert_psum[e] + out.expert_count[e];
            const int hi = (int)min((int64_t)out.expert_psum[e + 1], p.recv_capacity);
            for (int s = lo + tid; s < hi; s += nthreads) out.recv_src_token_idx[s] = -1;
        }
    }
}

int bits_for(int n) {  // bits needed to tell apart n distinct ids
    int b = 0;
    while ((1 << b) < n) ++b;
    return b;
}

template <typename IdxT>
hipError_t launch_typed(const LayoutParams& p, const TileGeometry& g, const void* topk,
                        const dispatch_layout_t& out, void* workspace, hipStream_t stream) {
    auto* hdr = reinterpret_cast<WorkspaceHeader*>(workspace);
    auto* tile_hist = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kWorkspaceHeader);
    auto* tile_base = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kWorkspaceHeader + g.hist_bytes);
    const auto* idx = static_cast<const IdxT*>(topk);
    const dim3 grid(g.num_tiles), block(g.waves_per_tile * kWave);
    const size_t lds = (size_t)g.waves_per_tile * g.num_keys * sizeof(int);
    LayoutParams pc = p;
    dispatch_layout_t oc = out;
    void* count_args[] = {&idx, &pc, &hdr, &tile_hist, &tile_base, &oc};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&count_kernel<IdxT>), grid, block,
                                     count_args, lds, stream);
    if (err != hipSuccess) return err;
    const int32_t* base_c = tile_base;
    void* assign_args[] = {&idx, &pc, &base_c, &oc};
    return hipLaunchKernel(reinterpret_cast<const void*>(&assign_kernel<IdxT>), grid, block,
                           assign_args, lds, stream);
}

}  // namespace

hipError_t launch_layout(const dispatch_problem_t& prob, const TileGeometry& g, const void* topk_idx,
                         const dispatch_layout_t& out, void* workspace, hipStream_t stream) {
    LayoutParams p{};
    p.num_tokens = prob.num_tokens;
    p.recv_capacity = prob.recv_capacity_rows;
    p.rank_capacity = prob.rank_capacity_rows;
    p.num_topk = prob.num_topk;
    p.num_experts = prob.num_experts;
    p.num_ranks = prob.num_ranks;
    p.experts_per_rank = prob.num_experts / prob.num_ranks;
    p.alignment = prob.expert_alignment;
    p.expert_bits = bits_for(prob.num_experts);
    p.rank_bits = bits_for(prob.num_ranks);
    p.tokens_per_chunk = g.tokens_per_chunk;
    p.tokens_per_wave = g.tokens_per_wave;
    p.tokens_per_tile = g.tokens_per_tile;
    p.num_keys = g.num_keys;
    p.num_tiles = g.num_tiles;
    if (prob.topk_idx_bytes == 8) return launch_typed<int64_t>(p, g, topk_idx, out, workspace, stream);
    return launch_typed<int32_t>(p, g, topk_idx, out, workspace, stream);
}

}  // namespace moe_dispatch
