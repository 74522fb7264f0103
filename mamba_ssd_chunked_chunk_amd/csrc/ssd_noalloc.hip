// ssd_chunk_scan_noalloc: ssd_chunk_scan_ex for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid allocation).  The scan's scratch lives in one
// file-scope device array of SSD_SCRATCH_BYTES per GPU, which the code
// object brings with it when it is loaded on that GPU and which stays until
// the process ends.  Calls on one GPU share the array: calls that overlap
// (on different streams, or from different threads) race on it.  The scan
// never reads scratch it has not written in the same call, so nothing needs
// clearing between calls.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/ssd.h"

namespace {

__device__ __align__(256) unsigned char scratch[SSD_SCRATCH_BYTES];

// The array's device address on each device (its host-side name is only a
// stand-in, never a device address), looked up once per device with that
// device current.
constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_ptr[kMaxDevices];

hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" int32_t ssd_chunk_scan_noalloc(
    const void *x, const void *dt, const float *A, const void *B, const void *C,
    const float *D, const float *dt_bias, int32_t dt_softplus, float dt_min, float dt_max,
    const float *init_state, const int32_t *seq_idx, void *y, float *final_state,
    float *chunk_states, int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
    int64_t state_dim, int64_t groups, int64_t chunk, int32_t io_dtype, void *hip_stream,
    void *const *kernel_events) {
    // 0 for invalid sizes: ssd_chunk_scan_ex then reports them without
    // touching the scratch
    const size_t need = ssd_chunk_scan_workspace_bytes(batch, seqlen, heads, head_dim,
                                                       state_dim, groups, chunk);
    if (need > (size_t)SSD_SCRATCH_BYTES) return SSD_ERR_SCRATCH;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0 && batch > 0 && seqlen > 0) {
        if (scratch_address(&ws) != hipSuccess) return SSD_ERR_HIP;
        ws_bytes = (size_t)SSD_SCRATCH_BYTES;
    }
    return ssd_chunk_scan_ex(x, dt, A, B, C, D, dt_bias, dt_softplus, dt_min, dt_max,
                             init_state, seq_idx, y, final_state, chunk_states, batch, seqlen,
                             heads, head_dim, state_dim, groups, chunk, io_dtype, ws, ws_bytes,
                             hip_stream, kernel_events);
}
