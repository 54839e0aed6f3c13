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
// The routing table is cut into small tiles so that the whole GPU takes part
// (ranking a chunk is VALU work, and one CU would serialize a large tile).
// Up to three kernels, none of which waits on another workgroup:
//
//   count_kernel    one workgroup per tile: each wavefront ranks its chunks
//                   (see rank_chunk) into wavefront-private LDS counters; the
//                   tile's histogram row (one count per key) and its error
//                   bits go to the workspace.
//   colscan_kernel  (many tiles only) one workgroup per 64 keys: exclusive
//                   prefix of every histogram column over the tiles, and the
//                   column totals.
//   assign_kernel   one workgroup per tile: takes the column prefixes and
//                   totals (or, with few tiles, reduces the tile histograms
//                   itself), scans the totals into the aligned exclusive psums
//                   and the status (the same in every workgroup; workgroup 0
//                   stores them), ranks the tile's pairs again exactly as
//                   count_kernel did, and writes expert_slot, rank_slot and the
//                   inverse maps; pad entries of recv_src_token_idx become -1.
//
// Kernel boundaries order every hand-off; the workspace carries nothing from
// one call to the next and needs no clearing.
//
// Rank dedup: among the lanes of one token, the pair that owns a rank is the
// highest k in that rank (the page's "master lane"). gfx950 has no match-any
// instruction, so lanes holding equal keys are found with one ballot per key
// bit (a wavefront multisplit).
#include "dispatch_common.hpp"
#include "dispatch_device.hpp"

namespace moe_dispatch {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

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
    int32_t hist_stride;  // ints per histogram row (num_keys padded to a multiple of 4)
    int32_t num_tiles;
    int32_t exchange_words;  // one-launch layout: exchange words per tile
    int32_t exchange_sum_run;  // words summed whole before their counts are split
    int64_t wait_limit;      // one-launch layout: polls before a tile gives up
    // Receiver-side expand only: the table is a fixed-stride receive buffer
    // of rows_per_source rows per source, source s holding recv_count[s]
    // rows; its expert ids are global, this receiver owns
    // [first_expert, first_expert + num_experts).
    const int32_t* recv_count;
    int32_t rows_per_source;
    int32_t first_expert;
    int32_t global_experts;
    // Read-ahead of the token rows (the combined layout-and-scatter call
    // only): workgroups [num_tiles, num_tiles + pf_groups) of the launch read
    // the 16-byte vectors [pf_rows_lo, pf_rows_hi) of x and the words
    // [pf_sf_lo, pf_sf_hi) of x_sf and discard them.
    const u32x4* pf_rows;
    const uint32_t* pf_sf;
    int64_t pf_rows_lo, pf_rows_hi;
    int64_t pf_sf_lo, pf_sf_hi;
    int32_t pf_groups;
};

// Where one lane's pair lands inside its wavefront's chunks.
struct PairPos {
    int expert;      // expert id, or -1 when the lane holds no routed pair
    int expert_pos;  // earlier pairs of that expert in the wavefront's chunks
    int rank;        // rank id when the lane owns its (token, rank), else -1
    int rank_pos;    // earlier owned (token, rank) pairs of that rank in the wavefront's chunks
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
// beyond the chunk or the table). `counters` holds the wavefront's running
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
    const uint64_t own_token = ((1ull << K) - 1ull) << (token_in_chunk * K);
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

// Loads this lane's entry of each of the wavefront's chunks. With EXPAND,
// the entry is seen from the receiver: rows past their source's count are
// masked, another rank's experts are masked, local experts are renumbered
// from 0 and an id >= the global expert count becomes num_experts, which
// rank_chunk reports as a bad expert.
template <int CH, bool EXPAND, typename IdxT>
__device__ __forceinline__ void load_entries(const IdxT* __restrict__ topk, int64_t wave_tok0, int token_in_chunk,
                                             int k, const LayoutParams& p, int64_t (&entry)[CH], uint32_t& err) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t tok = wave_tok0 + (int64_t)c * p.tokens_per_chunk + token_in_chunk;
        const bool live = token_in_chunk < p.tokens_per_chunk && tok < p.num_tokens;
        int64_t v = live ? (int64_t)topk[tok * p.num_topk + k] : -1;
        if (EXPAND && live) {
            const int64_t src = tok / p.rows_per_source;
            const int64_t row = tok - src * p.rows_per_source;
            const int count = p.recv_count[src];
            if (count < 0 || count > p.rows_per_source) err |= DISPATCH_STATUS_BAD_COUNT;
            if (row >= count) v = -1;
            else if (v >= p.global_experts) v = p.num_experts;
            else if (v >= 0) v = (v >= p.first_expert && v < p.first_expert + p.num_experts) ? v - p.first_expert : -1;
        }
        entry[c] = v;
    }
}

// Inclusive sum over the 64 lanes of a wavefront through DPP moves, which
// stay in the vector unit (a shuffle is an LDS instruction and waits LDS
// latency at every step): shifts within each row of 16 lanes, then the last
// lane of row 0 and of row 2 added to rows 1 and 3, then lane 31 added to
// rows 2 and 3. Rows a move does not write keep 0 from `old`. (Measured on
// MI355X in the one-launch layout: 0.3 us less per scan than shuffles.)
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 1, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 2, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 4, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 8, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowBcast15, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kRowBcast31, 0xc, 0xf, false);
    return x;
}

// Two exclusive scans in one pass by the whole workgroup: of in[0, n_a),
// each value rounded up to a multiple of `align` first, and of in[n_a, n),
// each starting from 0, both into out. Returns the two totals. `scratch`
// holds 2 * wavefronts ints. Every wavefront scans the wavefront totals
// itself (lane w holding wavefront w's), so one barrier separates the two
// levels.
__device__ int2 block_exclusive_scan2(const int* __restrict__ in, int* __restrict__ out, int n_a, int n, int align,
                                      int* __restrict__ scratch) {
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = nthreads / kWave;
    const int per = (n + nthreads - 1) / nthreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int la = 0, lb = 0;
    for (int i = lo; i < hi; ++i) {
        const int c = in[i];
        if (i < n_a) la += align > 1 ? (c + align - 1) / align * align : c;
        else lb += c;
    }
    const int ia = wave_inclusive_sum(la), ib = wave_inclusive_sum(lb);
    if (lane == kWave - 1) {
        scratch[2 * wave] = ia;
        scratch[2 * wave + 1] = ib;
    }
    __syncthreads();
    const int sa = wave_inclusive_sum(lane < nwaves ? scratch[2 * lane] : 0);
    const int sb = wave_inclusive_sum(lane < nwaves ? scratch[2 * lane + 1] : 0);
    const int w = __builtin_amdgcn_readfirstlane(wave), last = __builtin_amdgcn_readfirstlane(nwaves - 1);
    const int before_a = w > 0 ? __builtin_amdgcn_readlane(sa, w > 0 ? w - 1 : 0) : 0;
    const int before_b = w > 0 ? __builtin_amdgcn_readlane(sb, w > 0 ? w - 1 : 0) : 0;
    int ra = before_a + ia - la, rb = before_b + ib - lb;
    for (int i = lo; i < hi; ++i) {
        const int c = in[i];
        if (i < n_a) {
            out[i] = ra;
            ra += align > 1 ? (c + align - 1) / align * align : c;
        } else {
            out[i] = rb;
            rb += c;
        }
    }
    const int2 totals = make_int2(__builtin_amdgcn_readlane(sa, last), __builtin_amdgcn_readlane(sb, last));
    __syncthreads();
    return totals;
}

// Workspace views.
struct Workspace {
    int32_t* tile_hist;    // [num_tiles][hist_stride]
    int32_t* tile_prefix;  // [num_tiles][hist_stride] pairs of the key in earlier tiles
    int32_t* totals;       // [num_keys]
    int32_t* tile_err;     // [num_tiles] DISPATCH_STATUS_* bits seen by the tile
    uint64_t* exchange;      // one-launch layout: [num_tiles][exchange_words] words of the exchange region
    uint64_t* exchange_ctl;  // its control word
};

// Read-ahead of the token rows while the layout runs. The layout kernels
// are chains of dependent latencies that leave HBM idle; the row scatter
// that follows reads every live token row once while it writes about
// fourteen times as many bytes. Reading the rows here, into the Infinity
// Cache, takes those reads out of the scatter's write stream: on MI355X a
// scatter whose rows come from HBM ran 18 us slower on the 4096 x 7168
// bf16 batch than one whose rows were already in the cache. Workgroup
// `group` of pf_groups reads one contiguous share of each range; the loaded
// values feed an empty asm statement, so the loads are kept but nothing is
// written.
__device__ __forceinline__ void read_ahead(const LayoutParams& p, int group) {
    constexpr int kInFlight = 16;  // 16-byte loads per thread issued before the first wait
    const int tid = threadIdx.x, nt = blockDim.x;
    const int G = p.pf_groups;
    uint32_t acc = 0;
    {
        const int64_t n = p.pf_rows_hi - p.pf_rows_lo, per = (n + G - 1) / G;
        const int64_t lo = p.pf_rows_lo + group * per, hi = min(p.pf_rows_hi, lo + per);
        // Indices past the share are clamped to its last vector: a repeated
        // load costs nothing, and every load is issued unconditionally.
        for (int64_t i = lo + tid; i < hi; i += (int64_t)kInFlight * nt) {
            u32x4 v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) v[u] = p.pf_rows[min(i + (int64_t)u * nt, hi - 1)];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    {
        const int64_t n = p.pf_sf_hi - p.pf_sf_lo, per = (n + G - 1) / G;
        const int64_t lo = p.pf_sf_lo + group * per, hi = min(p.pf_sf_hi, lo + per);
        for (int64_t i = lo + tid; i < hi; i += (int64_t)kInFlight * nt) {
            uint32_t v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) v[u] = p.pf_sf[min(i + (int64_t)u * nt, hi - 1)];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
        }
    }
    asm volatile("" ::"v"(acc));
}

template <int CH, bool EXPAND, typename IdxT>
__global__ void __launch_bounds__(kLayoutThreads)
count_kernel(const IdxT* __restrict__ topk, LayoutParams p, Workspace ws) {
    extern __shared__ int lds[];  // [W][num_keys] wavefront counters
    __shared__ uint32_t block_err;
    if ((int)blockIdx.x >= p.num_tiles) {  // a read-ahead workgroup
        read_ahead(p, blockIdx.x - p.num_tiles);
        return;
    }

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nthreads = blockDim.x, nwaves = nthreads / kWave, nkeys = p.num_keys;
    int* counters = lds + wave * nkeys;
    for (int i = lane; i < nkeys; i += kWave) counters[i] = 0;
    if (tid == 0) block_err = 0;
    __syncthreads();

    const int token_in_chunk = lane / p.num_topk;
    const int k = lane - token_in_chunk * p.num_topk;
    const int64_t wave_tok0 = (int64_t)blockIdx.x * p.tokens_per_tile + (int64_t)wave * p.tokens_per_wave;
    int64_t entry[CH];
    uint32_t err = 0;
    load_entries<CH, EXPAND>(topk, wave_tok0, token_in_chunk, k, p, entry, err);
#pragma unroll
    for (int c = 0; c < CH; ++c) (void)rank_chunk(entry[c], lane, token_in_chunk, p, counters, err);
    uint32_t wave_err = 0;
    for (uint32_t bit = 1; bit <= DISPATCH_STATUS_BAD_COUNT; bit <<= 1)
        if (__ballot((err & bit) != 0)) wave_err |= bit;
    if (lane == 0 && wave_err) atomicOr(&block_err, wave_err);
    __syncthreads();

    int32_t* row = ws.tile_hist + (int64_t)blockIdx.x * p.hist_stride;
    for (int j = tid; j < p.hist_stride; j += nthreads) {
        int s = 0;
        if (j < nkeys)
            for (int w = 0; w < nwaves; ++w) s += lds[w * nkeys + j];
        row[j] = s;  // the row's padding holds zeros
    }
    if (tid == 0) ws.tile_err[blockIdx.x] = (int32_t)block_err;
}

// Column scan of the tile histograms. A workgroup takes kpb = min(64, keys)
// consecutive keys; its kScanThreads threads are (segment, key) pairs, the
// tiles split into kScanThreads / kpb contiguous segments.
__global__ void __launch_bounds__(kScanThreads)
colscan_kernel(LayoutParams p, Workspace ws, int kpb) {
    __shared__ int seg_sum[kScanThreads];
    const int nseg = kScanThreads / kpb;
    const int kk = threadIdx.x % kpb, seg = threadIdx.x / kpb;
    const bool active = seg < nseg;
    const int j = blockIdx.x * kpb + kk;
    const int nkeys = p.num_keys, n = p.num_tiles, stride = p.hist_stride;
    const int per = (n + nseg - 1) / nseg;
    const int lo = active ? min(n, seg * per) : n, hi = active ? min(n, lo + per) : n;
    // The first kColscanHeld tiles of a segment stay in registers between the
    // two passes; all loads of a pass are independent, so they overlap.
    constexpr int kColscanHeld = 8;
    int held[kColscanHeld];
    int s = 0;
    if (j < nkeys) {
#pragma unroll
        for (int q = 0; q < kColscanHeld; ++q) {
            held[q] = lo + q < hi ? ws.tile_hist[(int64_t)(lo + q) * stride + j] : 0;
            s += held[q];
        }
#pragma unroll 8
        for (int i = lo + kColscanHeld; i < hi; ++i) s += ws.tile_hist[(int64_t)i * stride + j];
    }
    if (active) seg_sum[seg * kpb + kk] = s;
    __syncthreads();
    if (!active) return;
    int run = 0;
    for (int q = 0; q < seg; ++q) run += seg_sum[q * kpb + kk];
    if (j < nkeys) {
#pragma unroll
        for (int q = 0; q < kColscanHeld; ++q) {
            if (lo + q < hi) {
                ws.tile_prefix[(int64_t)(lo + q) * stride + j] = run;
                run += held[q];
            }
        }
#pragma unroll 8
        for (int i = lo + kColscanHeld; i < hi; ++i) {
            const int h = ws.tile_hist[(int64_t)i * stride + j];
            ws.tile_prefix[(int64_t)i * stride + j] = run;
            run += h;
        }
        if (seg == nseg - 1) ws.totals[j] = run;
    }
}

// Rows for the one-launch small-batch dispatch (assign_kernel with FUSED):
// the token rows and the two output layouts, as dispatch_scatter takes them.
struct RowArgs {
    const u32x4* x;
    const uint32_t* x_sf;
    u32x4* rank_x;
    uint32_t* rank_sf;
    u32x4* recv_x;
    uint32_t* recv_sf;
    int64_t row_vecs;         // row_bytes / 16
    int32_t sf_per_token;
    int32_t segments;         // 1 KB units per row (64 vectors each)
    int32_t units_per_group;  // (token, unit) pairs each workgroup copies
    int32_t write_rank;       // rank_x / rank_sf requested
    int32_t write_expert;     // recv_x / recv_sf requested
    int32_t zero_pad;         // pad rows of recv_x / recv_sf zeroed
};

// Alignment pads of recv_src_token_idx (section 7.3): the slots after an
// expert's routed rows up to its aligned end map to no token. The experts
// are read 64 at a time, one per lane, and the ones with pad slots are
// shared out: the layout_groups workgroups' wavefronts are split evenly over
// the groups of 64 experts (or take several groups each when there are fewer
// wavefronts than groups), and wavefront `sub` of a group takes every
// per_group-th padded expert of it. All lanes then store that expert's
// slots. first[] holds the exclusive psums, totals[] the expert counts.
__device__ __forceinline__ void write_pad_entries(const LayoutParams& p, const int* first, const int* totals,
                                                  int recv_rows, int layout_groups, int group, int wave, int lane,
                                                  int nwaves, const dispatch_layout_t& out) {
    const int E = p.num_experts;
    const int groups = (E + kWave - 1) / kWave;
    const int stride = layout_groups * nwaves, me = group * nwaves + wave;
    const int per_group = stride > groups ? stride / groups : 1;
    const int sub = me % per_group;
    for (int g = me / per_group; g < groups; g += stride / per_group) {
        const int e = g * kWave + lane;
        int lo = 0, hi = 0;
        if (e < E) {
            lo = first[e] + totals[e];
            hi = (int)min((int64_t)(e + 1 < E ? first[e + 1] : recv_rows), p.recv_capacity);
        }
        const bool padded = hi > lo;
        const int rank = __popcll(__ballot(padded) & ((1ull << lane) - 1ull));
        for (uint64_t m = __ballot(padded && rank % per_group == sub); m != 0; m &= m - 1) {
            const int i = __builtin_ctzll(m);
            const int lo_i = __builtin_amdgcn_readlane(lo, i), hi_i = __builtin_amdgcn_readlane(hi, i);
            for (int s = lo_i + lane; s < hi_i; s += kWave) out.recv_src_token_idx[s] = -1;
        }
    }
}

// Where assign_kernel takes each key's count in earlier tiles and in all tiles:
enum AssignMode {
    kFromColumnScan = 0,  // the column-scan kernel's prefixes and totals
    kFromHistograms = 1,  // its own reduction of the count kernel's tile histograms
    kSingleTile = 2,      // one tile holds every pair: its own wavefront counters (no count kernel)
};

// FUSED (with kSingleTile only): the whole dispatch of a small batch in one
// launch. The batch is one tile of up to 8 chunks per wavefront, and every
// workgroup ranks the entire tile itself (a few microseconds of redundant ALU
// work, no communication between workgroups).
// Workgroup 0 writes the counts, psums and status. Workgroup g copies the row
// units [g * units_per_group, (g + 1) * units_per_group), a unit being one
// token's 1 KB row segment, to the token's destination rows; it writes the
// slot-map entries and scale factors of the tokens whose first unit it holds,
// and zeroes its share of the pad rows (chunks of an expert's consecutive pad
// rows, dealt round-robin over the workgroups). The results equal those of
// the layout followed by the scatter.
template <int CH, int MODE, bool EXPAND, typename IdxT, bool FUSED = false>
__global__ void __launch_bounds__(kLayoutThreads)
assign_kernel(const IdxT* __restrict__ topk, LayoutParams p, Workspace ws, dispatch_layout_t out, RowArgs rows) {
    static_assert(!FUSED || MODE == kSingleTile, "the fused dispatch ranks one tile");
    if (!FUSED && (int)blockIdx.x >= p.num_tiles) {  // a read-ahead workgroup
        read_ahead(p, blockIdx.x - p.num_tiles);
        return;
    }
    // LDS: [W][num_keys] wavefront counters, then totals[num_keys] and first[num_keys].
    extern __shared__ int lds[];
    __shared__ int scratch[2 * (kLayoutThreads / kWave + 1)];
    __shared__ uint32_t block_err;
    __shared__ int dest_expert[FUSED ? kFusedMaxPairs : 1], dest_rank[FUSED ? kFusedMaxPairs : 1];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nthreads = blockDim.x, nwaves = nthreads / kWave, nkeys = p.num_keys;
    const int K = p.num_topk, E = p.num_experts, R = p.num_ranks;
    const int tile = FUSED ? 0 : blockIdx.x;
    // The workgroup that writes the counts, psums and status.
    const bool writes_totals = FUSED ? blockIdx.x == 0 : tile == 0;
    // FUSED: this workgroup's row units [unit0, unit1) and the tokens they
    // belong to, [tok_first, tok_end).
    const int64_t segs = FUSED ? rows.segments : 1;
    const int64_t unit0 = FUSED ? min((int64_t)blockIdx.x * rows.units_per_group, p.num_tokens * segs) : 0;
    const int64_t unit1 = FUSED ? min(unit0 + rows.units_per_group, p.num_tokens * segs) : 0;
    const int64_t tok_first = unit0 / segs;
    const int64_t tok_end = unit1 > unit0 ? (unit1 - 1) / segs + 1 : tok_first;
    if constexpr (FUSED) {
        if (tid < kFusedMaxPairs) {
            dest_expert[tid] = -1;
            dest_rank[tid] = -1;
        }
    }
    int* counters = lds + wave * nkeys;
    int* totals = lds + nwaves * nkeys;  // per key, over all tiles
    int* first = totals + nkeys;         // per key, first slot (exclusive psum)
    // The routing entries and the tiles' error words do not depend on the
    // histograms: their loads go out first, so the three latencies overlap.
    const int token_in_chunk = lane / K;
    const int k = lane - token_in_chunk * K;
    const int64_t wave_tok0 = (int64_t)tile * p.tokens_per_tile + (int64_t)wave * p.tokens_per_wave;
    int64_t entry[CH];
    uint32_t err = 0;
    load_entries<CH, EXPAND>(topk, wave_tok0, token_in_chunk, k, p, entry, err);
    uint32_t tile_errs = 0;
    if (MODE != kSingleTile)
        for (int i = tid; i < p.num_tiles; i += nthreads) tile_errs |= (uint32_t)ws.tile_err[i];
    for (int i = lane; i < nkeys; i += kWave) counters[i] = 0;
    // totals[] holds each key's pair count over all tiles; first[] holds, for
    // now, its pairs in tiles before this one.
    if (MODE == kFromHistograms) {
        // Every thread sums 16-byte histogram pieces (4 keys) over a strided
        // set of tiles; the partial sums meet in LDS.
        for (int j = tid; j < nkeys; j += nthreads) {
            totals[j] = 0;
            first[j] = 0;
        }
        __syncthreads();
        // A thread's loads of one batch are all issued before the first add,
        // so a batch costs one memory latency.
        constexpr int kHistBatch = 16;
        const int quads = p.hist_stride / 4;
        const int groups = nthreads / quads > 1 ? nthreads / quads : 1;
        const i32x4* hist4 = reinterpret_cast<const i32x4*>(ws.tile_hist);
        for (int item = tid; item < quads * groups; item += nthreads) {
            const int q = item % quads, g = item / quads;
            i32x4 tot = {0, 0, 0, 0}, bef = {0, 0, 0, 0};
            for (int i0 = g; i0 < p.num_tiles; i0 += groups * kHistBatch) {
                i32x4 h[kHistBatch];
#pragma unroll
                for (int b = 0; b < kHistBatch; ++b) {
                    const int i = i0 + b * groups;
                    h[b] = i < p.num_tiles ? hist4[(int64_t)i * quads + q] : (i32x4){0, 0, 0, 0};
                }
#pragma unroll
                for (int b = 0; b < kHistBatch; ++b) {
                    tot += h[b];
                    if (i0 + b * groups < tile) bef += h[b];
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = 4 * q + c;
                if (j < nkeys && tot[c]) atomicAdd(&totals[j], tot[c]);
                if (j < nkeys && bef[c]) atomicAdd(&first[j], bef[c]);
            }
        }
    } else if (MODE == kFromColumnScan) {
        for (int j = tid; j < nkeys; j += nthreads) {
            totals[j] = ws.totals[j];
            first[j] = ws.tile_prefix[(int64_t)tile * p.hist_stride + j];
        }
    }
    if (tid == 0) block_err = 0;
    __syncthreads();
    if (tile_errs) atomicOr(&block_err, tile_errs);

    PairPos pos[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) pos[c] = rank_chunk(entry[c], lane, token_in_chunk, p, counters, err);
    if (MODE == kSingleTile) {
        // No count kernel ran: this workgroup's own ranking found the errors.
        uint32_t wave_err = 0;
        for (uint32_t bit = 1; bit <= DISPATCH_STATUS_BAD_COUNT; bit <<= 1)
            if (__ballot((err & bit) != 0)) wave_err |= bit;
        if (lane == 0 && wave_err) atomicOr(&block_err, wave_err);
    }

    // Fold the earlier-tile pairs into the wavefront counters, then scan the
    // totals into the exclusive psums: expert counts aligned up first
    // (section 7.2), rank counts as they are (section 5.2). The scan's
    // barriers also publish the wavefront counters and block_err. A single
    // tile has no earlier tiles, and its totals are its counters' sums.
    __syncthreads();
    for (int j = tid; j < nkeys; j += nthreads) {
        int run = MODE == kSingleTile ? 0 : first[j];
        for (int w = 0; w < nwaves; ++w) {
            const int c = lds[w * nkeys + j];
            lds[w * nkeys + j] = run;
            run += c;
        }
        if (MODE == kSingleTile) totals[j] = run;
    }
    if (MODE == kSingleTile) __syncthreads();
    const int2 row_totals = block_exclusive_scan2(totals, first, E, nkeys, p.alignment, scratch);
    const int recv_rows = row_totals.x, rank_rows = row_totals.y;
    uint32_t status = block_err;
    if (recv_rows > p.recv_capacity) status |= DISPATCH_STATUS_RECV_OVERFLOW;
    if (rank_rows > p.rank_capacity) status |= DISPATCH_STATUS_RANK_OVERFLOW;
    // The receiver-side expand has no rank outputs (their pointers are NULL).
    if (writes_totals) {
        for (int j = tid; j < nkeys; j += nthreads) {
            if (j < E) {
                out.expert_count[j] = totals[j];
                out.expert_psum[j] = first[j];
            } else if (out.rank_count) {
                out.rank_count[j - E] = totals[j];
                out.rank_psum[j - E] = first[j];
            }
        }
        // Running per-expert totals over calls, when asked for (section 7.2's
        // receive statistics): atomics, so concurrent calls may share them.
        if (status == 0 && out.expert_count_cumulative)
            for (int j = tid; j < E; j += nthreads) atomicAdd(&out.expert_count_cumulative[j], totals[j]);
        if (tid == 0) {
            out.expert_psum[E] = recv_rows;
            if (out.rank_psum) out.rank_psum[R] = rank_rows;
            *out.status = (int32_t)status;
        }
    }
    if (status != 0) return;  // the layout is unspecified: write nothing more

    // A pair's slot: its key's first slot, plus the key's pairs in earlier
    // tiles and earlier wavefronts of this tile (the counters), plus its rank
    // inside the wavefront's chunks.
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t tok = wave_tok0 + (int64_t)c * p.tokens_per_chunk + token_in_chunk;
        const bool live = token_in_chunk < p.tokens_per_chunk && tok < p.num_tokens;
        if (!live) continue;
        const int e = pos[c].expert, r = pos[c].rank;
        const int es = e >= 0 ? first[e] + counters[e] + pos[c].expert_pos : -1;
        const int rs = r >= 0 ? first[E + r] + counters[E + r] + pos[c].rank_pos : -1;
        if constexpr (FUSED) {
            // Every workgroup knows every slot. It keeps those of its tokens,
            // and writes the slot-map entries of the tokens whose first unit
            // is its own.
            if (tok < tok_first || tok >= tok_end) continue;
            dest_expert[(tok - tok_first) * K + k] = es;
            dest_rank[(tok - tok_first) * K + k] = rs;
            if (tok * segs < unit0) continue;
        }
        out.expert_slot[tok * K + k] = es;
        // Slots are below the totals, which fit the capacities when the
        // status is 0; the bounds are checked anyway before every store.
        if (es >= 0 && es < p.recv_capacity) out.recv_src_token_idx[es] = (int32_t)tok;
        if (out.rank_slot) {
            out.rank_slot[tok * K + k] = rs;
            if (rs >= 0 && rs < p.rank_capacity) out.rank_src_token_idx[rs] = (int32_t)tok;
        }
    }

    // Alignment pads of recv_src_token_idx, spread over the layout's
    // wavefronts. (One expert per wavefront loop step cost about 130 ns a
    // step: 33 us for a one-token layout over 256 experts, whose one tile has
    // one wavefront; one group of 64 experts per wavefront left most
    // wavefronts idle: 16 us for 257 tokens, against 11.)
    if (p.alignment > 1)
        write_pad_entries(p, first, totals, recv_rows, FUSED ? (int)gridDim.x : p.num_tiles, blockIdx.x, wave, lane,
                          nwaves, out);
    if constexpr (FUSED) {
        // The row copies of this workgroup's tokens (sections 6.3 and 8.2),
        // bitwise, each row read once: every thread takes 16-byte vectors of
        // the row and stores each to all of the token's destination rows.
        __syncthreads();
        const int64_t nv = rows.row_vecs;
        const int S = rows.sf_per_token;
        for (int64_t t = tok_first; t < tok_end; ++t) {
            const int64_t m = t - tok_first;
            // Slots past the capacities never occur with status 0; they are
            // dropped all the same, so no store can leave the output buffers.
            bool any = false;
            for (int kk = 0; kk < K; ++kk) {
                const int de = dest_expert[m * K + kk], dr = dest_rank[m * K + kk];
                any |= (rows.write_expert && de >= 0 && de < p.recv_capacity) ||
                       (rows.write_rank && dr >= 0 && dr < p.rank_capacity);
            }
            if (!any) continue;  // a row with no destination is not read
            // This workgroup's units of the row, as a range of 16-byte vectors.
            const int64_t u_lo = max(unit0, t * segs) - t * segs, u_hi = min(unit1, (t + 1) * segs) - t * segs;
            const int64_t v_hi = min(u_hi * kWave, nv);
            for (int64_t i = u_lo * kWave + tid; i < v_hi; i += nthreads) {
                const u32x4 v = rows.x[t * nv + i];
                for (int kk = 0; kk < K; ++kk) {
                    const int de = dest_expert[m * K + kk], dr = dest_rank[m * K + kk];
                    if (rows.write_expert && de >= 0 && de < p.recv_capacity)
                        RowWriter(rows.recv_x + (int64_t)de * nv, (int)(nv * 16)).store(i, v);
                    if (rows.write_rank && dr >= 0 && dr < p.rank_capacity)
                        RowWriter(rows.rank_x + (int64_t)dr * nv, (int)(nv * 16)).store(i, v);
                }
            }
            // The scale factors go with the row's first unit.
            for (int i = tid; i < (u_lo == 0 ? S : 0); i += nthreads) {
                const uint32_t v = rows.x_sf[t * S + i];
                for (int kk = 0; kk < K; ++kk) {
                    const int de = dest_expert[m * K + kk], dr = dest_rank[m * K + kk];
                    if (rows.write_expert && de >= 0 && de < p.recv_capacity) rows.recv_sf[(int64_t)de * S + i] = v;
                    if (rows.write_rank && dr >= 0 && dr < p.rank_capacity) rows.rank_sf[(int64_t)dr * S + i] = v;
                }
            }
        }
        // Pad rows are zero bytes (section 7.3). Expert e has at most A - 1 of
        // them, cut into chunks of kFusedPadChunk consecutive rows; the chunks
        // are dealt round-robin over all workgroups, so the pads of a few
        // experts still spread out. A workgroup finds its non-empty chunks 64
        // at a time, one per lane, numbers their rows in order and deals them
        // over its wavefronts, row q to wavefront q % nwaves: neighbouring
        // wavefronts write neighbouring rows, and no wavefront steps through
        // empty chunks one by one.
        if (rows.write_expert && rows.zero_pad && p.alignment > 1) {
            const u32x4 zero = {0u, 0u, 0u, 0u};
            const int my_wave = __builtin_amdgcn_readfirstlane(wave);
            const int64_t chunks = (p.alignment - 1 + kFusedPadChunk - 1) / kFusedPadChunk;
            const int64_t mine = ((int64_t)E * chunks - blockIdx.x + gridDim.x - 1) / gridDim.x;
            int done = 0;  // rows of this workgroup's earlier non-empty chunks
            for (int64_t j0 = 0; j0 < mine; j0 += kWave) {
                int lo = 0, n = 0;
                if (j0 + lane < mine) {
                    const int64_t c = blockIdx.x + (j0 + lane) * gridDim.x;
                    const int e = (int)(c / chunks);
                    lo = first[e] + totals[e] + (int)(c - e * chunks) * kFusedPadChunk;
                    const int end = (int)min((int64_t)(e + 1 < E ? first[e + 1] : recv_rows), p.recv_capacity);
                    n = max(0, min(kFusedPadChunk, end - lo));
                }
                for (uint64_t m = __ballot(n > 0); m != 0; m &= m - 1) {
                    const int i = __builtin_ctzll(m);
                    const int lo_i = __builtin_amdgcn_readlane(lo, i), n_i = __builtin_amdgcn_readlane(n, i);
                    for (int r = (my_wave - done % nwaves + nwaves) % nwaves; r < n_i; r += nwaves) {
                        const int64_t row = (int64_t)lo_i + r;
                        const RowWriter dst(rows.recv_x + row * nv, (int)(nv * 16));
                        for (int64_t v = lane; v < nv; v += kWave) dst.store(v, zero);
                        for (int v = lane; v < S; v += kWave) rows.recv_sf[row * S + v] = 0u;
                    }
                    done += n_i;
                }
            }
        }
    }
}

// One-launch layout: Count, Prefix Sum and the slot assignment of a batch of
// several tiles in a single kernel, for the layouts that read the token rows
// ahead (the combined call, dispatch_layout_read_ahead). Workgroup `tile`
// ranks its tile's pairs once (rank_chunk), keeping each pair's place in
// registers, and publishes the tile's key counts and error bits as exchange
// words: relaxed agent-scope atomic stores with bit 63 set. It then reads
// every tile's words until all of them are published (relaxed agent-scope
// atomic loads; each word is written once per call and carries its own
// "published" bit, so no ordering between locations is needed), summing the
// key totals and the counts of earlier tiles as it reads, and assigns its
// slots exactly as assign_kernel does. A tile holds fewer than 4096 (token,
// k) pairs, so each of its counts fits the 12 bits a word gives it. Workgroups past the tiles read the
// token rows ahead, all of them.
// The tiles are the first workgroups of the grid and wait on nothing but
// each other, so all of them are resident while they wait (the wait is
// bounded all the same: a tile that gives up writes nothing and the call
// reports DISPATCH_STATUS_TIMEOUT). Once a tile has read every word (or
// given up) and knows the status, it makes one atomic add on the control
// word (tiles done, tiles that gave up, tile 0's status bits); the last one
// writes the status and clears the words and the control word, so the next
// call finds them zero.
constexpr uint64_t kPublished = uint64_t(1) << 63;
constexpr uint64_t kCountMask = (uint64_t(1) << kExchangeCountBits) - 1;
constexpr int kExchangeBatch = 16;  // exchange words a thread loads before it waits

template <int CH, typename IdxT>
__global__ void __launch_bounds__(kLayoutThreads)
exchange_layout_kernel(const IdxT* __restrict__ topk, LayoutParams p, Workspace ws, dispatch_layout_t out) {
    if ((int)blockIdx.x >= p.num_tiles) {  // a read-ahead workgroup
        read_ahead(p, blockIdx.x - p.num_tiles);
        return;
    }
    // LDS: [W][num_keys] wavefront counters, then totals[num_keys],
    // first[num_keys] and own[num_keys].
    extern __shared__ int lds[];
    __shared__ int scratch[2 * (kLayoutThreads / kWave + 1)];
    __shared__ uint32_t block_err;
    __shared__ int last_tile;
    constexpr int kMaxWaves = kLayoutThreads / kWave;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nthreads = blockDim.x, nwaves = nthreads / kWave, nkeys = p.num_keys;
    const int K = p.num_topk, E = p.num_experts, R = p.num_ranks;
    const int tile = blockIdx.x;
    int* counters = lds + wave * nkeys;
    int* totals = lds + nwaves * nkeys;  // per key, over all tiles
    int* first = totals + nkeys;         // per key: pairs in earlier tiles
    int* own = first + nkeys;            // per key: this tile's pairs, then the key's first slot
    const int token_in_chunk = lane / K;
    const int k = lane - token_in_chunk * K;
    const int64_t wave_tok0 = (int64_t)tile * p.tokens_per_tile + (int64_t)wave * p.tokens_per_wave;
    int64_t entry[CH];
    uint32_t err = 0;
    load_entries<CH, false>(topk, wave_tok0, token_in_chunk, k, p, entry, err);
    for (int i = lane; i < nkeys; i += kWave) counters[i] = 0;
    for (int j = tid; j < nkeys; j += nthreads) {
        totals[j] = 0;
        first[j] = 0;
    }
    if (tid == 0) block_err = 0;
    __syncthreads();

    PairPos pos[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) pos[c] = rank_chunk(entry[c], lane, token_in_chunk, p, counters, err);
    {
        uint32_t wave_err = 0;
        for (uint32_t bit = 1; bit <= DISPATCH_STATUS_BAD_COUNT; bit <<= 1)
            if (__ballot((err & bit) != 0)) wave_err |= bit;
        if (lane == 0 && wave_err) atomicOr(&block_err, wave_err);
    }
    __syncthreads();

    // Publish the tile's count of every key, kExchangeCountsPerWord to a
    // word, then its error bits. The counts are summed over the wavefronts
    // first, one key per thread, so the words all go out after one LDS
    // round. (Measured on MI355X: packing the words straight from the
    // wavefront counters, 5 keys times 8 wavefronts read in turn by each of
    // 53 threads, took 1.8 us, and every other tile waited for it; this
    // takes 0.9 us.)
    for (int j = tid; j < nkeys; j += nthreads) {
        int c[kMaxWaves];
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) c[w] = w < nwaves ? lds[w * nkeys + j] : 0;
        int sum = 0;
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) sum += c[w];
        own[j] = sum;
    }
    __syncthreads();
    const int wpt = p.exchange_words;
    const int qwords = wpt - 1;
    uint64_t* mine = ws.exchange + (int64_t)tile * wpt;
    for (int q = tid; q < wpt; q += nthreads) {
        uint64_t v = kPublished;
        if (q < qwords) {
#pragma unroll
            for (int c = 0; c < kExchangeCountsPerWord; ++c) {
                const int j = q * kExchangeCountsPerWord + c;
                if (j < nkeys) v |= ((uint64_t)own[j] & kCountMask) << (c * kExchangeCountBits);
            }
        } else {
            v |= block_err;
        }
        __hip_atomic_store(mine + q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // While the other tiles publish, each wavefront counter becomes the
    // key's pairs in the tile's earlier wavefronts (last read by the sums
    // above, before the barrier); the slots add the earlier tiles' pairs and
    // the key's first slot once the exchange is done.
    for (int j = tid; j < nkeys; j += nthreads) {
        int c[kMaxWaves];
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) c[w] = w < nwaves ? lds[w * nkeys + j] : 0;
        int run = 0;
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) {
            if (w < nwaves) lds[w * nkeys + j] = run;
            run += c[w];
        }
    }

    // Every tile's words, until all are published. Each round reads the
    // words this thread has not yet found published: the error words (each
    // tile's last) of tiles tid, tid + threads, ..., and count word q of
    // group g's tiles, a run of consecutive tiles (qwords <= threads per
    // tile; at most 64 tiles per group). A word is written once per call, so
    // once published its value is final, and it is added the first time it
    // is found. Readiness is decided per word, never inferred from another
    // word. (Measured on MI355X, flushed steps, against reading only the
    // error words until all were there and then every count word: the
    // aligned fp8 batch, 64 tiles, 0.8-1.2 us faster; the metric batch, bound
    // by its read-ahead, and the Zipf batch, 256 tiles, the same within
    // 0.5 us. Reading the count words of a tile only after a round had found
    // its error word, for 64 tiles or for more, gained nothing.)
    const int groups = nthreads / qwords;
    const int q = tid % qwords, g = tid / qwords;
    const int per_group = (p.num_tiles + groups - 1) / groups;
    const int t0 = g * per_group;
    const int my_tiles = g < groups ? max(0, min(per_group, p.num_tiles - t0)) : 0;
    uint64_t todo = my_tiles >= 64 ? ~uint64_t(0) : (uint64_t(1) << my_tiles) - 1;  // my tiles not yet added
    uint32_t err_todo = 0;  // error words of tiles tid, tid + nthreads, ... not yet seen
    for (int b = 0; b * nthreads + tid < p.num_tiles; ++b) err_todo |= 1u << b;
    int tot[kExchangeCountsPerWord] = {}, bef[kExchangeCountsPerWord] = {};
    const int run_mask = p.exchange_sum_run - 1;
    uint32_t errs = 0;
    bool timed_out = false;
    for (int64_t poll = 0;; ++poll) {
        if (poll == p.wait_limit) {
            timed_out = true;
            break;
        }
        const uint64_t need = todo;
        // The error words are loaded first and looked at last, so that one
        // memory round trip serves both kinds of word.
        constexpr int kErrPerThread = kExchangeMaxTiles / kWave;  // tiles <= 256, threads >= 64
        uint64_t ev[kErrPerThread];
#pragma unroll
        for (int b = 0; b < kErrPerThread; ++b)
            ev[b] = ((err_todo >> b) & 1u) ? __hip_atomic_load(ws.exchange + (int64_t)(b * nthreads + tid) * wpt + qwords,
                                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                           : 0;
        for (int m0 = 0; m0 < my_tiles && (need >> m0) != 0; m0 += kExchangeBatch) {
            uint64_t v[kExchangeBatch];
#pragma unroll
            for (int b = 0; b < kExchangeBatch; ++b) {
                const int m = m0 + b;
                v[b] = m < my_tiles && ((need >> m) & 1)
                           ? __hip_atomic_load(ws.exchange + (int64_t)(t0 + m) * wpt + q, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0;
            }
            // The words are summed as 64-bit integers, run_mask + 1 at a
            // time, and only the sums split into counts. (Measured on
            // MI355X: splitting every word, 16 x 5 counts per thread, made a
            // round 0.3 us longer.)
            uint64_t sum_all = 0, sum_before = 0;
#pragma unroll
            for (int b = 0; b < kExchangeBatch; ++b) {
                if (v[b] & kPublished) {
                    const uint64_t w = v[b] & ~kPublished;
                    sum_all += w;
                    if (t0 + m0 + b < tile) sum_before += w;
                    todo &= ~(uint64_t(1) << (m0 + b));
                }
                if (((b + 1) & run_mask) == 0) {
#pragma unroll
                    for (int c = 0; c < kExchangeCountsPerWord; ++c) {
                        tot[c] += (int)((sum_all >> (c * kExchangeCountBits)) & kCountMask);
                        bef[c] += (int)((sum_before >> (c * kExchangeCountBits)) & kCountMask);
                    }
                    sum_all = sum_before = 0;
                }
            }
        }
#pragma unroll
        for (int b = 0; b < kErrPerThread; ++b) {
            if (ev[b] & kPublished) {
                errs |= (uint32_t)ev[b];
                err_todo &= ~(1u << b);
            }
        }
        if (!__syncthreads_or(todo != 0 || err_todo != 0)) break;
        __builtin_amdgcn_s_sleep(2);
    }

    uint32_t status = 0;
    int recv_rows = 0;
    if (!timed_out) {
        if (g < groups) {
#pragma unroll
            for (int c = 0; c < kExchangeCountsPerWord; ++c) {
                const int j = q * kExchangeCountsPerWord + c;
                if (j < nkeys && tot[c]) atomicAdd(&totals[j], tot[c]);
                if (j < nkeys && bef[c]) atomicAdd(&first[j], bef[c]);
            }
        }
        if (errs) atomicOr(&block_err, errs);
        __syncthreads();
        // The totals scanned into the exclusive psums (expert counts aligned
        // up first), each key's first slot, into own[] (free since the words
        // went out).
        const int2 row_totals = block_exclusive_scan2(totals, own, E, nkeys, p.alignment, scratch);
        recv_rows = row_totals.x;
        const int rank_rows = row_totals.y;
        status = block_err;
        if (recv_rows > p.recv_capacity) status |= DISPATCH_STATUS_RECV_OVERFLOW;
        if (rank_rows > p.rank_capacity) status |= DISPATCH_STATUS_RANK_OVERFLOW;
        if (tile == 0) {
            for (int j = tid; j < nkeys; j += nthreads) {
                if (j < E) {
                    out.expert_count[j] = totals[j];
                    out.expert_psum[j] = own[j];
                } else {
                    out.rank_count[j - E] = totals[j];
                    out.rank_psum[j - E] = own[j];
                }
            }
            if (status == 0 && out.expert_count_cumulative)
                for (int j = tid; j < E; j += nthreads) atomicAdd(&out.expert_count_cumulative[j], totals[j]);
            if (tid == 0) {
                out.expert_psum[E] = recv_rows;
                out.rank_psum[R] = rank_rows;
            }
        }
    }

    // This tile is done with the exchange: count it in the control word
    // (bits [0, 24): tiles done; [24, 48): tiles that gave up; [48, 64):
    // tile 0's status bits). The reply is awaited only after the tile's slot
    // writes. The last tile to count itself (every tile has read every word
    // by then) writes the status and clears the words and the control word
    // for the next call. (Measured on MI355X: with the counters folded during
    // the wait as well, the layout of the aligned fp8 batch, 64 tiles, ends
    // 0.5 us sooner than when each tile awaited the reply first.)
    uint64_t ctl_add = 1, ctl_old = 0;
    if (tid == 0) {
        if (timed_out) ctl_add |= uint64_t(1) << 24;
        else if (tile == 0) ctl_add |= (uint64_t)(status & 0xffffu) << 48;
        ctl_old = __hip_atomic_fetch_add(ws.exchange_ctl, ctl_add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    if (!timed_out && status == 0) {  // else the layout is unspecified: no slots
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t tok = wave_tok0 + (int64_t)c * p.tokens_per_chunk + token_in_chunk;
            if (token_in_chunk >= p.tokens_per_chunk || tok >= p.num_tokens) continue;
            const int e = pos[c].expert, r = pos[c].rank;
            const int es = e >= 0 ? own[e] + first[e] + counters[e] + pos[c].expert_pos : -1;
            const int rs = r >= 0 ? own[E + r] + first[E + r] + counters[E + r] + pos[c].rank_pos : -1;
            out.expert_slot[tok * K + k] = es;
            if (es >= 0 && es < p.recv_capacity) out.recv_src_token_idx[es] = (int32_t)tok;
            out.rank_slot[tok * K + k] = rs;
            if (rs >= 0 && rs < p.rank_capacity) out.rank_src_token_idx[rs] = (int32_t)tok;
        }
        if (p.alignment > 1) write_pad_entries(p, own, totals, recv_rows, p.num_tiles, tile, wave, lane, nwaves, out);
    }

    if (tid == 0) {
        last_tile = (int)((ctl_old & 0xffffffu) + 1 == (uint64_t)p.num_tiles);
        if (last_tile) {
            const uint64_t all = ctl_old + ctl_add;
            uint32_t st = (uint32_t)(all >> 48);
            if ((all >> 24) & 0xffffffu) st |= DISPATCH_STATUS_TIMEOUT;
            *out.status = (int32_t)st;
        }
    }
    __syncthreads();
    if (last_tile) {
        const int64_t words = (int64_t)p.num_tiles * wpt;
        for (int64_t i = tid; i < words; i += nthreads) ws.exchange[i] = 0;
        if (tid == 0) *ws.exchange_ctl = 0;
    }
}

int bits_for(int n) {  // bits needed to tell apart n distinct ids
    int b = 0;
    while ((1 << b) < n) ++b;
    return b;
}

template <int CH, bool EXPAND, typename IdxT>
hipError_t launch_typed(const LayoutParams& p, const TileGeometry& g, const void* topk,
                        const dispatch_layout_t& out, const Workspace& ws, hipStream_t stream,
                        const ReadAhead* ra) {
    const auto* idx = static_cast<const IdxT*>(topk);
    const dim3 grid(g.num_tiles), block(g.waves_per_tile * kWave);
    LayoutParams pc = p;
    Workspace wc = ws;
    dispatch_layout_t oc = out;
    RowArgs rc{};  // no rows: the layout alone
    const size_t assign_lds = (size_t)(g.waves_per_tile + 2) * g.num_keys * sizeof(int);
    void* assign_args[] = {&idx, &pc, &wc, &oc, &rc};
    if (g.num_tiles == 1 && !g.column_scan)
        return hipLaunchKernel(reinterpret_cast<const void*>(&assign_kernel<CH, kSingleTile, EXPAND, IdxT>), grid,
                               block, assign_args, assign_lds, stream);
    // Read-ahead shares: the count kernel takes the scale factors and the
    // first rows, the assign kernel (the longer of the two) the other rows.
    const bool reads_ahead = ra != nullptr && ra->x != nullptr && ra->x_bytes > 0;
    const int64_t row_vecs = reads_ahead ? ra->x_bytes / 16 : 0;
    const int64_t split = row_vecs * kReadAheadCountPct / 100;
    const dim3 ra_grid(g.num_tiles + (reads_ahead ? kReadAheadGroups : 0));
    if (reads_ahead) {
        pc.pf_rows = static_cast<const u32x4*>(ra->x);
        pc.pf_sf = reinterpret_cast<const uint32_t*>(ra->x_sf);
        pc.pf_rows_lo = 0;
        pc.pf_rows_hi = split;
        pc.pf_sf_lo = 0;
        pc.pf_sf_hi = ra->x_sf != nullptr ? ra->sf_words : 0;
        pc.pf_groups = kReadAheadGroups;
    }
    const size_t count_lds = (size_t)g.waves_per_tile * g.num_keys * sizeof(int);
    void* count_args[] = {&idx, &pc, &wc};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&count_kernel<CH, EXPAND, IdxT>), ra_grid, block,
                                     count_args, count_lds, stream);
    if (err != hipSuccess) return err;
    if (reads_ahead) {  // hipLaunchKernel has copied the count kernel's arguments
        pc.pf_rows_lo = split;
        pc.pf_rows_hi = row_vecs;
        pc.pf_sf_lo = pc.pf_sf_hi = 0;
    }
    if (!g.column_scan)
        return hipLaunchKernel(reinterpret_cast<const void*>(&assign_kernel<CH, kFromHistograms, EXPAND, IdxT>),
                               ra_grid, block, assign_args, assign_lds, stream);
    int kpb = g.num_keys < kWave ? g.num_keys : kWave;
    void* scan_args[] = {&pc, &wc, &kpb};
    err = hipLaunchKernel(reinterpret_cast<const void*>(&colscan_kernel),
                          dim3((g.num_keys + kpb - 1) / kpb), dim3(kScanThreads), scan_args, 0, stream);
    if (err != hipSuccess) return err;
    return hipLaunchKernel(reinterpret_cast<const void*>(&assign_kernel<CH, kFromColumnScan, EXPAND, IdxT>), ra_grid,
                           block, assign_args, assign_lds, stream);
}

template <bool EXPAND, typename IdxT>
hipError_t launch_chunks(const LayoutParams& p, const TileGeometry& g, const void* topk,
                         const dispatch_layout_t& out, const Workspace& ws, hipStream_t stream,
                         const ReadAhead* ra) {
    switch (g.chunks_per_wave) {
        case 1: return launch_typed<1, EXPAND, IdxT>(p, g, topk, out, ws, stream, ra);
        case 2: return launch_typed<2, EXPAND, IdxT>(p, g, topk, out, ws, stream, ra);
        case 4: return launch_typed<4, EXPAND, IdxT>(p, g, topk, out, ws, stream, ra);
        default: return launch_typed<8, EXPAND, IdxT>(p, g, topk, out, ws, stream, ra);
    }
}

template <int CH, bool EXPAND, typename IdxT>
hipError_t launch_fused_typed(const LayoutParams& p, const TileGeometry& g, const void* topk,
                              const dispatch_layout_t& out, const Workspace& ws, const RowArgs& rows,
                              const FusedShape& f, hipStream_t stream) {
    const auto* idx = static_cast<const IdxT*>(topk);
    LayoutParams pc = p;
    Workspace wc = ws;
    dispatch_layout_t oc = out;
    RowArgs rc = rows;
    // f.waves may exceed the tile's wavefronts: the extra ones rank empty
    // chunks (no change to any count) and add their threads to the copies.
    const size_t lds = (size_t)(f.waves + 2) * g.num_keys * sizeof(int);
    void* args[] = {&idx, &pc, &wc, &oc, &rc};
    return hipLaunchKernel(reinterpret_cast<const void*>(&assign_kernel<CH, kSingleTile, EXPAND, IdxT, true>),
                           dim3((unsigned)f.groups), dim3(f.waves * kWave), args, lds, stream);
}

LayoutParams make_params(const dispatch_problem_t& prob, const TileGeometry& g) {
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
    p.hist_stride = g.hist_stride;
    p.num_tiles = g.num_tiles;
    p.exchange_words = g.exchange_words;
    p.exchange_sum_run = g.exchange_sum_run;
    return p;
}

Workspace make_workspace(const TileGeometry& g, void* workspace) {
    char* base = static_cast<char*>(workspace);
    Workspace ws;
    ws.tile_hist = reinterpret_cast<int32_t*>(base + g.ws_tile_hist);
    ws.tile_prefix = reinterpret_cast<int32_t*>(base + g.ws_tile_prefix);
    ws.totals = reinterpret_cast<int32_t*>(base + g.ws_totals);
    ws.tile_err = reinterpret_cast<int32_t*>(base + g.ws_tile_err);
    ws.exchange = reinterpret_cast<uint64_t*>(base + g.ws_exchange);
    ws.exchange_ctl = ws.exchange + kExchangeRegionWords;
    return ws;
}

}  // namespace

hipError_t launch_layout(const dispatch_problem_t& prob, const TileGeometry& g, const void* topk_idx,
                         const dispatch_layout_t& out, void* workspace, hipStream_t stream,
                         const ExpandView* expand, const ReadAhead* ra) {
    LayoutParams p = make_params(prob, g);
    const Workspace ws = make_workspace(g, workspace);
    if (expand != nullptr) {
        p.recv_count = expand->recv_count;
        p.rows_per_source = expand->rows_per_source;
        p.first_expert = expand->first_expert;
        p.global_experts = expand->global_experts;
        if (prob.topk_idx_bytes == 8) return launch_chunks<true, int64_t>(p, g, topk_idx, out, ws, stream, ra);
        return launch_chunks<true, int32_t>(p, g, topk_idx, out, ws, stream, ra);
    }
    if (prob.topk_idx_bytes == 8) return launch_chunks<false, int64_t>(p, g, topk_idx, out, ws, stream, ra);
    return launch_chunks<false, int32_t>(p, g, topk_idx, out, ws, stream, ra);
}


namespace {

template <int CH, bool EXPAND>
hipError_t launch_fused_width(bool wide, const LayoutParams& p, const TileGeometry& tile, const void* topk,
                              const dispatch_layout_t& out, const Workspace& ws, const RowArgs& rows,
                              const FusedShape& f, hipStream_t stream) {
    return wide ? launch_fused_typed<CH, EXPAND, int64_t>(p, tile, topk, out, ws, rows, f, stream)
                : launch_fused_typed<CH, EXPAND, int32_t>(p, tile, topk, out, ws, rows, f, stream);
}

template <bool EXPAND>
hipError_t launch_fused_chunks(bool wide, const LayoutParams& p, const TileGeometry& tile, const void* topk,
                               const dispatch_layout_t& out, const Workspace& ws, const RowArgs& rows,
                               const FusedShape& f, hipStream_t stream) {
    switch (f.chunks) {
        case 1: return launch_fused_width<1, EXPAND>(wide, p, tile, topk, out, ws, rows, f, stream);
        case 2: return launch_fused_width<2, EXPAND>(wide, p, tile, topk, out, ws, rows, f, stream);
        case 4: return launch_fused_width<4, EXPAND>(wide, p, tile, topk, out, ws, rows, f, stream);
        default: return launch_fused_width<8, EXPAND>(wide, p, tile, topk, out, ws, rows, f, stream);
    }
}

}  // namespace

hipError_t launch_fused_dispatch(const dispatch_problem_t& prob, const TileGeometry& g, const void* topk_idx,
                                 const dispatch_layout_t& out, void* workspace, const void* x, const float* x_sf,
                                 void* rank_x, float* rank_sf, void* recv_x, float* recv_sf, hipStream_t stream,
                                 const ExpandView* expand) {
    const FusedShape f = fused_shape(prob, g, expand != nullptr);
    if (!f.fits) return hipErrorInvalidValue;
    // The one tile every workgroup ranks (the layout's own geometry may use
    // several tiles for this batch).
    TileGeometry tile = g;
    tile.chunks_per_wave = f.chunks;
    tile.waves_per_tile = f.tile_waves;
    tile.tokens_per_wave = f.chunks * g.tokens_per_chunk;
    tile.tokens_per_tile = f.tile_waves * tile.tokens_per_wave;
    tile.num_tiles = 1;
    tile.column_scan = false;
    LayoutParams p = make_params(prob, tile);
    if (expand != nullptr) {
        p.recv_count = expand->recv_count;
        p.rows_per_source = expand->rows_per_source;
        p.first_expert = expand->first_expert;
        p.global_experts = expand->global_experts;
    }
    const Workspace ws = make_workspace(g, workspace);
    RowArgs rows{};
    rows.x = static_cast<const u32x4*>(x);
    rows.x_sf = reinterpret_cast<const uint32_t*>(x_sf);
    rows.rank_x = static_cast<u32x4*>(rank_x);
    rows.rank_sf = reinterpret_cast<uint32_t*>(rank_sf);
    rows.recv_x = static_cast<u32x4*>(recv_x);
    rows.recv_sf = reinterpret_cast<uint32_t*>(recv_sf);
    rows.row_vecs = prob.row_bytes / 16;
    rows.sf_per_token = prob.sf_per_token;
    rows.segments = f.segments;
    rows.units_per_group = f.units_per_group;
    rows.write_rank = (prob.flags & DISPATCH_RANK_CONTIG) != 0;
    rows.write_expert = (prob.flags & DISPATCH_EXPERT_MAJOR) != 0;
    rows.zero_pad = (prob.flags & DISPATCH_ZERO_PAD) != 0;
    const bool wide = prob.topk_idx_bytes == 8;
    if (expand != nullptr) return launch_fused_chunks<true>(wide, p, tile, topk_idx, out, ws, rows, f, stream);
    return launch_fused_chunks<false>(wide, p, tile, topk_idx, out, ws, rows, f, stream);
}

namespace {

template <int CH, typename IdxT>
hipError_t launch_exchange_typed(const LayoutParams& p, const TileGeometry& g, const void* topk,
                                 const dispatch_layout_t& out, const Workspace& ws, hipStream_t stream) {
    const auto* idx = static_cast<const IdxT*>(topk);
    LayoutParams pc = p;
    Workspace wc = ws;
    dispatch_layout_t oc = out;
    void* args[] = {&idx, &pc, &wc, &oc};
    const size_t lds = (size_t)(g.waves_per_tile + 3) * g.num_keys * sizeof(int);
    return hipLaunchKernel(reinterpret_cast<const void*>(&exchange_layout_kernel<CH, IdxT>),
                           dim3((unsigned)(g.num_tiles + p.pf_groups)), dim3(g.waves_per_tile * kWave), args, lds,
                           stream);
}

}  // namespace

bool exchange_layout_fits(const dispatch_problem_t& prob, const TileGeometry& g) {
    // Exchange room in the geometry, a thread per count word of a tile, and
    // at most 64 tiles for each group of threads that reads a tile's words.
    if (g.exchange_words <= 0 || prob.num_tokens <= 0) return false;
    const int threads = g.waves_per_tile * kWave, qwords = g.exchange_words - 1;
    if (qwords > threads) return false;
    const int groups = threads / qwords;
    return (g.num_tiles + groups - 1) / groups <= 64;
}

hipError_t launch_exchange_layout(const dispatch_problem_t& prob, const TileGeometry& g, const void* topk_idx,
                                  const dispatch_layout_t& out, void* workspace, const ReadAhead* ra,
                                  hipStream_t stream) {
    if (!exchange_layout_fits(prob, g)) return hipErrorInvalidValue;
    LayoutParams p = make_params(prob, g);
    p.wait_limit = exchange_wait_limit();
    if (ra != nullptr && (ra->x_bytes > 0 || ra->sf_words > 0)) {
        p.pf_rows = static_cast<const u32x4*>(ra->x);
        p.pf_sf = reinterpret_cast<const uint32_t*>(ra->x_sf);
        p.pf_rows_lo = 0;
        p.pf_rows_hi = ra->x != nullptr ? ra->x_bytes / 16 : 0;
        p.pf_sf_lo = 0;
        p.pf_sf_hi = ra->x_sf != nullptr ? ra->sf_words : 0;
        p.pf_groups = exchange_read_ahead_groups(p.pf_rows_hi * 16 + p.pf_sf_hi * 4);
    }
    const Workspace ws = make_workspace(g, workspace);
    const bool wide = prob.topk_idx_bytes == 8;
#define MOE_DISPATCH_EXCHANGE_CASE(N)                                                      \
    case N:                                                                                \
        return wide ? launch_exchange_typed<N, int64_t>(p, g, topk_idx, out, ws, stream) \
                    : launch_exchange_typed<N, int32_t>(p, g, topk_idx, out, ws, stream);
    switch (g.chunks_per_wave) {
        MOE_DISPATCH_EXCHANGE_CASE(1)
        MOE_DISPATCH_EXCHANGE_CASE(2)
        MOE_DISPATCH_EXCHANGE_CASE(4)
        MOE_DISPATCH_EXCHANGE_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef MOE_DISPATCH_EXCHANGE_CASE
}

}  // namespace moe_dispatch
