// Allocation-free form of dispatch_layout_and_scatter.
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the layout
// kernels' workspace (per-tile histograms, prefixes, key totals and error
// words) lives in a file-scope device array of a fixed size instead of a
// caller-provided buffer. Each GPU the library runs on holds its own copy of
// the array until the process ends. The workspace is rewritten before it is
// read on every call, so nothing in it needs clearing; calls that overlap in
// time on one GPU share the array and race.
#include <mutex>

#include "dispatch_common.hpp"
#include "moe_dispatch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[DISPATCH_NOALLOC_WORKSPACE_BYTES];

// The array's device address, looked up once per device with that device
// current. In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies take the looked-up address only.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];
std::once_flag g_once[kMaxDevices];

hipError_t scratch_on(int device, void** out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[device], [device] {
        int current = 0;
        hipError_t err = hipGetDevice(&current);
        if (err == hipSuccess && current != device) err = hipSetDevice(device);
        void* ptr = nullptr;
        if (err == hipSuccess) err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (current != device) (void)hipSetDevice(current);
        g_lookup[device] = err;
        g_scratch[device] = err == hipSuccess ? ptr : nullptr;
    });
    *out = g_scratch[device];
    return g_lookup[device];
}

}  // namespace

extern "C" int dispatch_layout_and_scatter_noalloc(const dispatch_problem_t* problem, const void* topk_idx,
                                                   const dispatch_layout_t* out, const void* x, const float* x_sf,
                                                   void* rank_x, float* rank_sf, void* recv_x, float* recv_sf,
                                                   hipStream_t stream) {
    size_t need = 0;
    const int rc = dispatch_workspace_size(problem, &need);
    if (rc != DISPATCH_OK) return rc;
    if (need > sizeof(scratch)) return DISPATCH_ERR_WORKSPACE;  // beyond the fixed array: refused
    int device = 0;
    if ((stream != nullptr ? hipStreamGetDevice(stream, &device) : hipGetDevice(&device)) != hipSuccess)
        return DISPATCH_ERR_HIP;
    void* ws = nullptr;
    if (scratch_on(device, &ws) != hipSuccess || ws == nullptr) return DISPATCH_ERR_HIP;
    return dispatch_layout_and_scatter(problem, topk_idx, out, ws, sizeof(scratch), x, x_sf, rank_x, rank_sf,
                                       recv_x, recv_sf, stream);
}
