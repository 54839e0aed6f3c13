// Internal definitions shared by the dispatch kernels and their host launchers.
//
// Tile geometry of the layout pass. The routing table is cut into tiles of
// consecutive tokens, one workgroup per tile. A workgroup holds W wavefronts;
// wavefront w owns a sub-tile of CHUNKS chunks, and a chunk packs
// floor(64 / K) tokens x K top-k entries into the 64 lanes of a wavefront, one
// lane per (token, k) pair, in (token, k) order. Processing chunks in order
// inside a wavefront, sub-tiles in order inside a tile and tiles in order
// inside the batch walks the pairs in ascending token order, which is what
// makes the slots stable without any order-dependent atomics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dispatch.h"

namespace moe_dispatch {

constexpr int kWave = 64;            // gfx950 wavefront width
constexpr int kChunksPerWave = 8;    // chunks per wavefront sub-tile
constexpr int kMaxWavesPerTile = 16; // 1024-thread workgroups
constexpr int kLdsBudgetInts = 16000; // per-wavefront key counters, under 64 KiB of LDS
constexpr size_t kWorkspaceHeader = 256;

// Workspace control words (zero between calls; the last workgroup of the
// count kernel resets them).
struct WorkspaceHeader {
    uint32_t ticket;     // workgroups of the count kernel that have finished
    uint32_t error_bits; // DISPATCH_STATUS_* bits raised by any workgroup
};

struct TileGeometry {
    int64_t num_tokens;
    int32_t num_topk;
    int32_t tokens_per_chunk;   // floor(64 / K)
    int32_t tokens_per_wave;    // tokens_per_chunk * kChunksPerWave
    int32_t waves_per_tile;     // W
    int32_t tokens_per_tile;    // W * tokens_per_wave
    int32_t num_tiles;          // >= 1
    int32_t num_keys;           // E + R: expert keys first, then rank keys
    size_t hist_bytes;          // one [num_tiles][num_keys] int32 table, 256-byte padded
};

inline size_t round_up_256(size_t v) { return (v + 255) & ~size_t(255); }

inline TileGeometry make_geometry(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                                  int32_t num_ranks) {
    TileGeometry g{};
    g.num_tokens = num_tokens;
    g.num_topk = num_topk;
    g.tokens_per_chunk = kWave / num_topk;
    g.tokens_per_wave = g.tokens_per_chunk * kChunksPerWave;
    g.num_keys = num_experts + num_ranks;
    int w = kLdsBudgetInts / g.num_keys;
    g.waves_per_tile = w < 1 ? 1 : (w > kMaxWavesPerTile ? kMaxWavesPerTile : w);
    g.tokens_per_tile = g.waves_per_tile * g.tokens_per_wave;
    int64_t tiles = (num_tokens + g.tokens_per_tile - 1) / g.tokens_per_tile;
    g.num_tiles = tiles < 1 ? 1 : (int32_t)tiles;
    g.hist_bytes = round_up_256((size_t)g.num_tiles * (size_t)g.num_keys * sizeof(int32_t));
    return g;
}

// Workspace: [header | tile_hist[num_tiles][num_keys] | tile_base[num_tiles][num_keys]].
inline size_t workspace_bytes(const TileGeometry& g) { return kWorkspaceHeader + 2 * g.hist_bytes; }

// Launchers (defined in the .hip files). They return the HIP error of the launch.
hipError_t launch_layout(const dispatch_problem_t& p, const TileGeometry& g, const void* topk_idx,
                         const dispatch_layout_t& out, void* workspace, hipStream_t stream);
hipError_t launch_scatter(const dispatch_problem_t& p, const dispatch_layout_t& lay, const void* x,
                          const float* x_sf, void* rank_x, float* rank_sf, void* recv_x,
                          float* recv_sf, hipStream_t stream);

}  // namespace moe_dispatch
