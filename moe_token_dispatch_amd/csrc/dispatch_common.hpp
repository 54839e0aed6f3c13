// Internal definitions shared by the dispatch kernels and their host launchers.
//
// Tile geometry of the layout pass. The routing table is cut into tiles of
// consecutive tokens, one workgroup per tile. A workgroup holds W wavefronts;
// wavefront w owns CH consecutive chunks, and a chunk packs floor(64 / K)
// tokens x K top-k entries into the 64 lanes of a wavefront, one lane per
// (token, k) pair, in (token, k) order. Ranking chunks in order inside a
// wavefront, wavefronts in order inside a tile and tiles in order inside the
// batch walks the pairs in ascending token order, which is what makes the
// slots stable without any order-dependent atomics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dispatch.h"

namespace moe_dispatch {

constexpr int kWave = 64;             // gfx950 wavefront width
constexpr int kLayoutThreads = 1024;  // at most 16 wavefronts per layout workgroup
constexpr int kScanThreads = 1024;    // threads per column-scan workgroup
constexpr int kMaxTilesTarget = 512;  // more chunks per wavefront beyond this many tiles
constexpr int kFromHistMaxInts = 65536;  // up to this many histogram ints, assign reduces them itself
constexpr int kSingleTileChunks = 2;     // most chunks per wavefront of a one-launch single tile
constexpr int kFewTileWaves = 16;     // wavefronts per tile on the two-launch path (at most)
constexpr int kMidTileWaves = 8;      // wavefronts per tile on the two-launch path when the histograms fit
constexpr int kManyTileWaves = 4;     // wavefronts per tile on the column-scan path
constexpr int kLdsBudgetInts = 40000; // LDS ints per workgroup for key arrays (gfx950: 160 KiB per CU)
constexpr int kLdsPerCu = 160 * 1024;  // gfx950
// Dynamic LDS per workgroup that lets at most n workgroups of a launch share
// a CU (a kernel that needs no LDS reserves it only to bound its occupancy):
// midway between the sizes at which n and n + 1 workgroups just fit, so that
// an allocation granularity of up to 2 KiB cannot change the count for
// n <= 8 (above that it may admit one workgroup fewer).
inline int lds_for_workgroups_per_cu(int n) {
    if (n < 1) n = 1;
    return (kLdsPerCu / n + kLdsPerCu / (n + 1)) / 2;
}

struct TileGeometry {
    int64_t num_tokens;
    int32_t num_topk;
    int32_t tokens_per_chunk;   // floor(64 / K)
    int32_t chunks_per_wave;    // CH: 1, 2, 4 or 8
    int32_t tokens_per_wave;    // tokens_per_chunk * CH
    int32_t waves_per_tile;     // W
    int32_t max_waves;          // the most wavefronts per workgroup the LDS budget allows (at most 16)
    int32_t tokens_per_tile;    // W * tokens_per_wave
    int32_t num_tiles;          // >= 1
    int32_t num_keys;           // E + R: expert keys first, then rank keys
    int32_t hist_stride;        // ints per histogram row: num_keys rounded up to a multiple of 4
    bool column_scan;           // false: two kernels (count, assign); true: count, colscan, assign
    size_t ws_tile_hist;        // workspace byte offsets of the arrays below
    size_t ws_tile_prefix;
    size_t ws_totals;
    size_t ws_tile_err;
    size_t ws_exchange;         // the one-launch layout's exchange region (see below): always at 0
    int32_t exchange_words;     // 64-bit exchange words per tile (0: no one-launch layout)
    int32_t exchange_sum_run;   // exchange words summed whole before their counts are split (1..16)
    size_t ws_bytes;
};

// One-launch layout (exchange_layout_kernel): the tiles of one launch hand
// their key counts to each other through 64-bit words in the workspace: per
// tile, ceil(keys / 5) words of five 12-bit counts and one word of error
// bits, each with bit 63 set once published. They live in a region of
// kExchangeRegionWords words and a control word at the start of every
// workspace (dispatch and expand alike), which no other kernel writes; the
// words are zero between calls (each call clears the ones it used when it
// ends), so a workspace must be zero-filled before its first use. Tiles
// hold at most 4095 (token, k) pairs (a count per key and tile fits 12 bits
// whatever the routing), and a launch has at most kExchangeMaxTiles of them,
// all resident at once.
constexpr int kExchangeCountsPerWord = 5;
constexpr int kExchangeCountBits = 12;
constexpr int kExchangeMaxTiles = 256;
constexpr int64_t kExchangeRegionWords = 8192;
constexpr size_t kExchangeRegionBytes = (size_t)(kExchangeRegionWords + 1) * sizeof(uint64_t);
// The wait bound of the next one-launch layouts (dispatch_set_wait_limit).
int64_t exchange_wait_limit();

inline size_t round_up_256(size_t v) { return (v + 255) & ~size_t(255); }

inline TileGeometry make_geometry(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                                  int32_t num_ranks) {
    TileGeometry g{};
    g.num_tokens = num_tokens;
    g.num_topk = num_topk;
    g.tokens_per_chunk = kWave / num_topk;
    g.num_keys = num_experts + num_ranks;
    // The assign kernel holds W wavefront counter rows plus two more rows of
    // num_keys ints in LDS.
    const int w_lds = kLdsBudgetInts / g.num_keys - 2;
    auto clamp_w = [&](int cap) { return w_lds < 1 ? 1 : (w_lds > cap ? cap : w_lds); };
    // Histogram rows are padded to whole 16-byte vectors.
    g.hist_stride = (g.num_keys + 3) / 4 * 4;
    // One launch when a single tile holds the batch: one chunk per wavefront
    // and just enough wavefronts, else 16 wavefronts of kSingleTileChunks.
    // Two launches while the tile histograms stay small (every assign
    // workgroup reduces them itself; a launch costs a few microseconds, more
    // than that reduction): 8-wavefront tiles, else 16-wavefront tiles of 1,
    // 2, 4 or 8 chunks per wavefront, the fewest that fit. Otherwise tiles of
    // 4 wavefronts and a column-scan kernel, with more chunks per wavefront
    // once the tile count would make the column scan long. (Measured on
    // MI355X: 8-wavefront tiles lay out 512 to 8192 tokens fastest.)
    const int w_full = clamp_w(kFewTileWaves);
    g.max_waves = w_full;
    const int64_t tpc = g.tokens_per_chunk;
    auto tiles_of = [&](int w, int ch) { return (num_tokens + (int64_t)w * ch * tpc - 1) / ((int64_t)w * ch * tpc); };
    g.column_scan = true;
    if (num_tokens <= (int64_t)w_full * tpc) {
        const int64_t need = (num_tokens + tpc - 1) / tpc;
        g.waves_per_tile = need < 1 ? 1 : (int32_t)need;
        g.chunks_per_wave = 1;
        g.column_scan = false;
    } else if (num_tokens <= (int64_t)w_full * kSingleTileChunks * tpc) {
        g.waves_per_tile = w_full;
        g.chunks_per_wave = kSingleTileChunks;
        g.column_scan = false;
    } else {
        const int w_mid = clamp_w(kMidTileWaves);
        g.chunks_per_wave = 1;
        if (tiles_of(w_mid, 1) * g.hist_stride <= kFromHistMaxInts) {
            g.waves_per_tile = w_mid;
            g.column_scan = false;
        } else {
            g.waves_per_tile = w_full;
            for (int ch = 1; ch <= 8; ch *= 2) {
                if (tiles_of(w_full, ch) * g.hist_stride <= kFromHistMaxInts) {
                    g.chunks_per_wave = ch;
                    g.column_scan = false;
                    break;
                }
            }
        }
    }
    if (g.column_scan) {
        g.chunks_per_wave = 1;
        g.waves_per_tile = clamp_w(kManyTileWaves);
        while (g.chunks_per_wave < 8) {
            const int64_t per_tile = (int64_t)g.waves_per_tile * g.chunks_per_wave * g.tokens_per_chunk;
            if ((num_tokens + per_tile - 1) / per_tile <= kMaxTilesTarget) break;
            g.chunks_per_wave *= 2;
        }
    }
    g.tokens_per_wave = g.tokens_per_chunk * g.chunks_per_wave;
    g.tokens_per_tile = g.waves_per_tile * g.tokens_per_wave;
    const int64_t tiles = (num_tokens + g.tokens_per_tile - 1) / g.tokens_per_tile;
    g.num_tiles = tiles < 1 ? 1 : (int32_t)tiles;
    const size_t table = round_up_256((size_t)g.num_tiles * (size_t)g.hist_stride * sizeof(int32_t));
    g.ws_exchange = 0;
    g.ws_tile_hist = round_up_256(kExchangeRegionBytes);
    g.ws_tile_prefix = g.ws_tile_hist + table;
    g.ws_totals = g.ws_tile_prefix + table;
    g.ws_tile_err = g.ws_totals + round_up_256((size_t)g.num_keys * sizeof(int32_t));
    g.ws_bytes = g.ws_tile_err + round_up_256((size_t)g.num_tiles * sizeof(int32_t));
    const int words = (g.num_keys + kExchangeCountsPerWord - 1) / kExchangeCountsPerWord + 1;
    // (The exchange kernel holds one more row of num_keys ints in LDS than
    // the assign kernel: the tile's own counts.)
    // A tile holds tokens_per_tile * K pairs, so no count of a key in it
    // can exceed that, even where a token repeats an expert.
    const int64_t tile_pairs = g.tokens_per_tile * (int64_t)num_topk;
    const bool exchange = !g.column_scan && g.num_tiles > 1 && g.num_tiles <= kExchangeMaxTiles &&
                          tile_pairs < (1 << kExchangeCountBits) &&
                          (int64_t)g.num_tiles * words <= kExchangeRegionWords &&
                          (int64_t)(g.waves_per_tile + 3) * g.num_keys <= kLdsBudgetInts;
    g.exchange_words = exchange ? words : 0;
    // This many words add up as plain 64-bit integers without one 12-bit
    // count carrying into the next: the most, up to 16, a power of two, with
    // run * tile_pairs < 2^12.
    int run = 16;
    while (run > 1 && run * tile_pairs >= (1 << kExchangeCountBits)) run /= 2;
    g.exchange_sum_run = exchange ? run : 0;
    return g;
}

// Workspace: the exchange region (kExchangeRegionWords words and a control
// word, uint64), then tile_hist[num_tiles][hist_stride],
// tile_prefix[num_tiles][hist_stride], totals[num_keys] and
// tile_err[num_tiles], int32, each 256-byte aligned.
inline size_t workspace_bytes(const TileGeometry& g) { return g.ws_bytes; }

// How the receiver-side expand sees its receive buffer through the layout
// kernels (see dispatch_expand_layout).
struct ExpandView {
    const int32_t* recv_count;  // [num_sources] rows each source sent
    int32_t rows_per_source;    // receive-buffer rows per source
    int32_t first_expert;       // first global expert id owned by this receiver
    int32_t global_experts;     // E of the sending side
};

// Token rows that the layout kernels of a combined layout-and-scatter call
// read ahead, into the Infinity Cache, for the scatter that follows: extra
// workgroups of the count kernel read the first share, those of the assign
// kernel the rest. Up to kReadAheadMaxBytes (rows and scale factors
// together; larger batches are not read ahead: they would push their own
// first rows out of the 256 MB cache before the scatter reads them).
struct ReadAhead {
    const void* x;
    int64_t x_bytes;     // a multiple of 16
    const float* x_sf;
    int64_t sf_words;
};
constexpr int64_t kReadAheadMaxBytes = int64_t(160) << 20;
constexpr int kReadAheadGroups = 256;     // read-ahead workgroups per layout kernel
constexpr int kReadAheadCountPct = 35;    // percent of the rows the count kernel reads
// Read-ahead workgroups of the one-launch layout, which reads all the rows:
// about 512 KB each, at least 160 and at most 512 of them. Measured on
// MI355X (flushed steps): 59 MB of rows read fastest by 160-176 workgroups
// (with the 64 tiles, 28-30 workgroups on each XCD's 32 CUs; 128 or 144:
// 1.1-1.6 us slower, 96: 2.7 us; before the exchange read its words as they
// were published, 512 was 2 us and 64 was 6 us slower than 128), 134 MB by
// 256 (128 or 512: 5 us slower).
constexpr int64_t kExchangeReadAheadBytesPerGroup = int64_t(512) << 10;
constexpr int kExchangeReadAheadMinGroups = 160;
constexpr int kExchangeReadAheadMaxGroups = 512;
inline int exchange_read_ahead_groups(int64_t bytes) {
    const int64_t g = (bytes + kExchangeReadAheadBytesPerGroup - 1) / kExchangeReadAheadBytesPerGroup;
    return g < kExchangeReadAheadMinGroups ? kExchangeReadAheadMinGroups
                                           : (g > kExchangeReadAheadMaxGroups ? kExchangeReadAheadMaxGroups : (int)g);
}
inline bool read_ahead_fits(int64_t x_bytes, int64_t sf_words) {
    return x_bytes + 4 * sf_words <= kReadAheadMaxBytes;
}

// Launchers (defined in the .hip files). They return the HIP error of the launch.
hipError_t launch_layout(const dispatch_problem_t& p, const TileGeometry& g, const void* topk_idx,
                         const dispatch_layout_t& out, void* workspace, hipStream_t stream,
                         const ExpandView* expand = nullptr, const ReadAhead* read_ahead = nullptr);
// few_destinations: rows go to about one destination each (sets the segment width).
// Whether the scatter's grid fits one launch (at most 2^31 - 1 workgroups and
// 2^32 - 1 work-items); checked before anything of a call is enqueued.
bool scatter_grid_fits(const dispatch_problem_t& p, bool few_destinations);
hipError_t launch_scatter(const dispatch_problem_t& p, const dispatch_layout_t& lay, const void* x,
                          const float* x_sf, void* rank_x, float* rank_sf, void* recv_x,
                          float* recv_sf, hipStream_t stream, bool few_destinations);
// One-launch dispatch of a batch that fits one layout tile: layout and row
// copies in a single kernel (the assign kernel's fused mode). The row copies
// are cut into units of one token's 1 KB row segment; workgroup g copies units
// [g * units_per_group, (g + 1) * units_per_group), so the copies spread over
// many CUs even when there are few tokens.
constexpr int kFusedGroups = 256;         // at most this many workgroups
constexpr int kFusedMaxPairs = 64;        // (token, k) pairs whose slots one workgroup holds
constexpr int kFusedMaxChunks = 8;        // chunks per wavefront of the one tile every workgroup ranks
// The most (token, k) pairs of a batch the one kernel takes. Every workgroup
// ranks them all; measured on MI355X, beyond about 3072 pairs that costs more
// than the layout and scatter launches it saves (at 4096 pairs: 14.0 against
// 12.6 us for 256-byte rows, 29.2 against 29.6 us for 14 KB rows).
constexpr int64_t kFusedMaxBatchPairs = 3072;
// A lower limit where the one kernel's own copies are light against its
// ranking: a batch with zero pad rows to write (the scatter's one-row pad
// wavefronts write them faster), and the receiver-side expand (about one
// destination per row). Measured on MI355X: with alignment 128 on 7 KB rows,
// 384 tokens took 61.0 us in one kernel against 58.0 in the layout and
// scatter kernels (256 tokens: 55.5 against 56.9); the expand of 8 sources
// took 14.6 against 13.2 us at 3072 entries of bf16 rows (10.4 against 10.8
// at 2048). Past 2048 pairs at top-8 every wavefront ranks 4 chunks.
constexpr int64_t kFusedMaxBatchPairsPadsOrExpand = 2048;
// The most (expert, pad row) items, E * (A - 1), the one kernel walks, and
// the consecutive pad rows it deals to a workgroup at a time.
constexpr int64_t kFusedMaxPadItems = int64_t(1) << 20;
constexpr int kFusedPadChunk = 8;
constexpr int kFusedStoresPerThread = 8;  // 16-byte stores per thread that size the wavefront count
struct FusedShape {
    bool fits;
    int32_t chunks;      // chunks per wavefront of the tile
    int32_t tile_waves;  // wavefronts the tile needs
    int64_t groups;
    int32_t units_per_group;
    int32_t segments;    // 1 KB units per row
    int32_t waves;       // wavefronts per workgroup (>= tile_waves)
};
// expand: the problem is a receiver-side expand seen as a dispatch.
inline FusedShape fused_shape(const dispatch_problem_t& prob, const TileGeometry& g, bool expand = false) {
    FusedShape f{};
    const int64_t t = g.num_tokens;
    const int64_t row_bytes = prob.row_bytes;
    // Zeroed pad rows: up to A - 1 per expert, dealt over all the workgroups.
    const bool pads = (prob.flags & DISPATCH_EXPERT_MAJOR) && (prob.flags & DISPATCH_ZERO_PAD) &&
                      prob.expert_alignment > 1;
    const int64_t pad_items = pads ? (int64_t)prob.num_experts * (prob.expert_alignment - 1) : 0;
    // The tile: the fewest chunks per wavefront that fit the batch in the
    // wavefronts LDS allows, then just enough wavefronts.
    const int64_t tpc = g.tokens_per_chunk;
    f.chunks = 1;
    while (f.chunks < kFusedMaxChunks && (int64_t)g.max_waves * f.chunks * tpc < t) f.chunks *= 2;
    const int64_t per_wave = (int64_t)f.chunks * tpc;
    const int64_t tw = (t + per_wave - 1) / per_wave;
    f.tile_waves = (int32_t)(tw < 1 ? 1 : tw);
    const int64_t vecs = row_bytes / 16;
    f.segments = (int32_t)(vecs < 1 ? 1 : (vecs + 63) / 64);
    const int64_t units = t * f.segments;
    // At least half a row per workgroup (measured on MI355X: one 1 KB unit per
    // workgroup ranks the batch in too many workgroups at once for wide rows,
    // a whole row per workgroup leaves CUs idle).
    const int64_t per = (f.segments + 1) / 2;
    const int64_t want = (units + per - 1) / per;
    f.groups = want < 1 ? 1 : (want < kFusedGroups ? want : kFusedGroups);
    if (pads) f.groups = kFusedGroups;  // the pad rows need the whole GPU
    f.units_per_group = (int32_t)(units < 1 ? 1 : (units + f.groups - 1) / f.groups);
    // A unit range touches at most this many tokens.
    const int64_t tokens = f.segments == 1 ? f.units_per_group : (f.units_per_group + f.segments - 1) / f.segments + 1;
    // Enough wavefronts for the copies (K expert rows and one rank row per
    // unit) and for this workgroup's share of the pad rows (only experts that
    // receive a pair have any: at most min(E, T*K) of them), at least those
    // the tile's ranking uses, at most what LDS allows.
    const int64_t unit_vecs = vecs < 64 ? vecs : 64;
    const int64_t pairs = t * g.num_topk;
    const int64_t pad_rows = pads ? (pairs < prob.num_experts ? pairs : prob.num_experts) *
                                        (prob.expert_alignment - 1) : 0;
    const int64_t stores = (int64_t)f.units_per_group * unit_vecs * (g.num_topk + 1) +
                           (pad_rows + f.groups - 1) / f.groups * (vecs < 1 ? 1 : vecs);
    int64_t w = (stores + kWave * kFusedStoresPerThread - 1) / (kWave * kFusedStoresPerThread);
    if (w > g.max_waves) w = g.max_waves;
    if (w < f.tile_waves) w = f.tile_waves;
    f.waves = (int32_t)w;
    const int64_t max_pairs = pads || expand ? kFusedMaxBatchPairsPadsOrExpand : kFusedMaxBatchPairs;
    f.fits = f.tile_waves <= g.max_waves && tokens * g.num_topk <= kFusedMaxPairs &&
             t * g.num_topk <= max_pairs && pad_items <= kFusedMaxPadItems;
    return f;
}
// Requires fused_shape(p, g).fits; the outputs are those of
// launch_layout followed by launch_scatter.
hipError_t launch_fused_dispatch(const dispatch_problem_t& p, const TileGeometry& g, const void* topk_idx,
                                 const dispatch_layout_t& out, void* workspace, const void* x, const float* x_sf,
                                 void* rank_x, float* rank_sf, void* recv_x, float* recv_sf, hipStream_t stream,
                                 const ExpandView* expand = nullptr);
// The one-launch layout of a dispatch: tiles that rank their pairs once,
// exchange their key counts through the workspace and assign their slots;
// with a read-ahead, the launch's other workgroups read the token rows
// ahead. exchange_layout_fits() tells whether a problem's geometry takes it;
// the outputs equal launch_layout's.
bool exchange_layout_fits(const dispatch_problem_t& p, const TileGeometry& g);
hipError_t launch_exchange_layout(const dispatch_problem_t& p, const TileGeometry& g, const void* topk_idx,
                                  const dispatch_layout_t& out, void* workspace, const ReadAhead* read_ahead,
                                  hipStream_t stream);
hipError_t launch_combine(int64_t num_tokens, int32_t num_topk, int64_t row_bytes, int64_t expert_rows,
                          const int32_t* expert_slot, const float* weights, const void* y, void* out,
                          hipStream_t stream);

}  // namespace moe_dispatch
