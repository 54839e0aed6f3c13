// Device-side helpers shared by the HIP kernels (included by .hip files only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_dispatch {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle) and two store cache policies: nt | sc1, streaming stores, the
// fastest form measured on MI355X for the scatter's rows, which are not read
// back here; sc1 alone, the fastest for the combine's single store per row.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kStreamingPolicy = 2 | 16;
constexpr int kSc1Policy = 16;

// Stores 16-byte vectors into one row of `row_bytes` bytes through a buffer
// resource spanning exactly that row: the hardware drops any store whose
// offset falls outside the row.
template <int kPolicy>
struct RowStore {
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ __forceinline__ RowStore(u32x4* row, int row_bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(row, 0, row_bytes, kBufferWord3)) {}
    __device__ __forceinline__ void store(int64_t vec, const u32x4& v) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)(vec * 16), 0, kPolicy);
    }
};
using RowWriter = RowStore<kStreamingPolicy>;

}  // namespace moe_dispatch
