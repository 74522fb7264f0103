// libssd.so host side: argument validation, launch planning, dispatch over
// the compiled (head_dim, state_dim) set, and the optional kernel timing.
// Nothing here allocates device memory: the caller passes every buffer.
#include <hip/hip_runtime.h>

#include <math.h>
#include <atomic>

#include "../../include/ssd.h"
#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

// ------------------------------------------------------ device queries ---
// Compute units per device, queried once per device id (the only state the
// library keeps; thread-safe).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 1;
    cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// -------------------------------------------------------------- dispatch ---
template <typename IO>
static hipError_t dispatch_scan(const ScanPlan &pl, const ScanArgs &a, hipStream_t s) {
#define SSD_CASE(PP, NN)                                                       \
    if (pl.p == PP && pl.n == NN) {                                            \
        if constexpr (sizeof(IO) == 2) return launch_scan16<PP, NN>(pl, a, s); \
        else return launch_scan<IO, PP, NN>(pl, a, s);                         \
    }
#define SSD_ROW(PP) SSD_CASE(PP, 32) SSD_CASE(PP, 64) SSD_CASE(PP, 128)
    SSD_ROW(16) SSD_ROW(32) SSD_ROW(64) SSD_ROW(128)
#undef SSD_ROW
#undef SSD_CASE
    return hipErrorInvalidValue;
}

template <typename IO>
static hipError_t dispatch_step(const StepArgs &a, hipStream_t s) {
#define SSD_CASE(PP, NN) \
    if (a.p == PP && a.n == NN) return launch_step<IO, PP, NN>(a, s);
#define SSD_ROW(PP) SSD_CASE(PP, 32) SSD_CASE(PP, 64) SSD_CASE(PP, 128)
    SSD_ROW(16) SSD_ROW(32) SSD_ROW(64) SSD_ROW(128)
#undef SSD_ROW
#undef SSD_CASE
    return hipErrorInvalidValue;
}

// final_state <- init_state (or zeros), for calls with nothing to scan.
__global__ void k_fill_state(float *__restrict__ dst, const float *__restrict__ src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// The fp32 scan on any compiled shape (the gradient pass runs its scans
// through this).
hipError_t scan_f32(const ScanPlan &pl, const ScanArgs &a, hipStream_t s) {
    return dispatch_scan<float>(pl, a, s);
}
hipError_t scan_bf16(const ScanPlan &pl, const ScanArgs &a, hipStream_t s) {
    return dispatch_scan<bf16>(pl, a, s);
}

static bool supported_dims(int64_t p, int64_t n) {
    return (p == 16 || p == 32 || p == 64 || p == 128) && (n == 32 || n == 64 || n == 128);
}
static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
static bool mul_ok(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= lim / a; }

}  // namespace ssd

namespace ssd {

// Every argument check of ssd_chunk_scan_ex, in its order (SSD_OK: the
// call launches); the mixer runs it before its first launch.
int32_t scan_status(const void *x, const void *dt, const float *A, const void *B, const void *C,
                    const float *D, const float *dt_bias, const float *init_state,
                    const int32_t *seq_idx, const void *y, const float *final_state,
                    const float *chunk_states, int64_t batch, int64_t seqlen, int64_t heads,
                    int64_t head_dim, int64_t state_dim, int64_t groups, int64_t chunk,
                    int32_t io_dtype, const void *workspace, size_t workspace_bytes) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || seqlen < 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0 ||
        groups <= 0 || chunk <= 0 || heads % groups != 0)
        return SSD_ERR_SHAPE;
    if (!supported_dims(head_dim, state_dim)) return SSD_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 62;
    if (!mul_ok(batch, seqlen, lim) || !mul_ok(batch * seqlen, heads, lim) ||
        !mul_ok(batch * seqlen * heads, 128 * 128, lim))
        return SSD_ERR_UNSUPPORTED;
    const bool work = batch > 0 && seqlen > 0;
    if (!A) return SSD_ERR_NULL;
    if (work && (!x || !dt || !B || !C || !y)) return SSD_ERR_NULL;
    const size_t es = io_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(dt, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(dt_bias, 4) ||
        !aligned(init_state, 16) || !aligned(final_state, 16) || !aligned(workspace, 256) ||
        !aligned(seq_idx, 4) || !aligned(chunk_states, 16))
        return SSD_ERR_ALIGN;
    if (!work) return SSD_OK;
    ScanPlan pl;
    if (!make_plan(pl, batch, seqlen, heads, head_dim, state_dim, groups, chunk, io_dtype))
        return SSD_ERR_SHAPE;
    // grid limits: one-dimensional grids of at most 2^31 - 1 workgroups
    const int64_t gmax = ((int64_t)1 << 31) - 1;
    if (pl.b * pl.nc * pl.h * 8 > gmax || pl.b * pl.h * pl.n * pl.p / 4 / 256 + 1 > gmax)
        return SSD_ERR_UNSUPPORTED;
    // 32-bit buffer offsets: 64 rows of x, B, C or y, and the padded rows of
    // one (batch, head)
    const int64_t lim32 = ((int64_t)1 << 31);
    if (64 * heads * head_dim * 4 >= lim32 || 64 * groups * state_dim * 4 >= lim32 ||
        pl.lp * 4 >= lim32)
        return SSD_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < ssd_chunk_scan_workspace_bytes(
                                            batch, seqlen, heads, head_dim, state_dim, groups,
                                            chunk))
        return SSD_ERR_WORKSPACE;
    return SSD_OK;
}

}  // namespace ssd

using namespace ssd;

extern "C" {

int32_t ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char *ssd_status_string(int32_t status) {
    switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL: return "a required pointer is NULL";
    case SSD_ERR_SHAPE: return "invalid sizes (negative or zero size, heads % groups != 0, "
                               "or chunk <= 0)";
    case SSD_ERR_UNSUPPORTED: return "unsupported head_dim / state_dim / io dtype or sizes "
                                     "beyond the launch limits";
    case SSD_ERR_WORKSPACE: return "workspace missing or smaller than "
                                   "ssd_chunk_scan_workspace_bytes()";
    case SSD_ERR_ALIGN: return "a pointer is not aligned as documented";
    case SSD_ERR_HIP: return "the HIP runtime reported an error at launch";
    case SSD_ERR_SCRATCH: return "the sizes need more scratch than SSD_SCRATCH_BYTES "
                                 "(use ssd_chunk_scan_ex with a workspace)";
    default: return "unknown status";
    }
}

size_t ssd_chunk_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads,
                                      int64_t head_dim, int64_t state_dim, int64_t groups,
                                      int64_t chunk) {
    ScanPlan pl;  // the layout does not depend on the io type
    if (!make_plan(pl, batch, seqlen, heads, head_dim, state_dim, groups, chunk, 0)) return 0;
    return pl.total;
}

int64_t ssd_chunk_scan_state_chunks(int64_t batch, int64_t seqlen, int64_t heads,
                                    int64_t head_dim, int64_t state_dim, int64_t groups,
                                    int64_t chunk, int32_t io_dtype, int32_t with_chunk_states) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    ScanPlan pl;
    if (!make_plan(pl, batch, seqlen, heads, head_dim, state_dim, groups, chunk, io_dtype))
        return SSD_ERR_SHAPE;
    if (!supported_dims(head_dim, state_dim)) return SSD_ERR_UNSUPPORTED;
    if (io_dtype == SSD_F32 || seqlen == 0) return pl.nc;
    // the caller's per-chunk states come from chunks of the caller's length
    // (or from the computed ones, stepped token by token)
    const bool per_chunk = with_chunk_states != 0;
    const int m = bf16_state_interval(pl, per_chunk, head_dim, true);
    return (pl.l + m * pl.Q - 1) / (m * pl.Q);
}

int32_t ssd_chunk_scan(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const float *dt_bias,
                       int32_t dt_softplus, float dt_min, float dt_max,
                       const float *init_state, void *y, float *final_state, int64_t batch,
                       int64_t seqlen, int64_t heads, int64_t head_dim, int64_t state_dim,
                       int64_t groups, int64_t chunk, int32_t io_dtype, void *workspace,
                       size_t workspace_bytes, void *hip_stream) {
    return ssd_chunk_scan_ex(x, dt, A, B, C, D, dt_bias, dt_softplus, dt_min, dt_max,
                             init_state, nullptr, y, final_state, nullptr, batch, seqlen,
                             heads, head_dim, state_dim, groups, chunk, io_dtype, workspace,
                             workspace_bytes, hip_stream, nullptr);
}

int32_t ssd_chunk_scan_ex(const void *x, const void *dt, const float *A, const void *B,
                          const void *C, const float *D, const float *dt_bias,
                          int32_t dt_softplus, float dt_min, float dt_max,
                          const float *init_state, const int32_t *seq_idx, void *y,
                          float *final_state, float *chunk_states, int64_t batch,
                          int64_t seqlen, int64_t heads, int64_t head_dim, int64_t state_dim,
                          int64_t groups, int64_t chunk, int32_t io_dtype, void *workspace,
                          size_t workspace_bytes, void *hip_stream, void *const *kernel_events) {
    const int32_t st = scan_status(x, dt, A, B, C, D, dt_bias, init_state, seq_idx, y,
                                   final_state, chunk_states, batch, seqlen, heads, head_dim,
                                   state_dim, groups, chunk, io_dtype, workspace,
                                   workspace_bytes);
    if (st != SSD_OK) return st;
    const bool work = batch > 0 && seqlen > 0;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);

    if (!work) {
        if (final_state && batch > 0) {
            const int64_t cnt = batch * heads * head_dim * state_dim;
            hipLaunchKernelGGL(k_fill_state, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s,
                               final_state, init_state, cnt);
            if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
        }
        return SSD_OK;
    }

    ScanPlan pl;
    make_plan(pl, batch, seqlen, heads, head_dim, state_dim, groups, chunk, io_dtype);

    ScanArgs a{x, dt, B, C, A, D, dt_bias, dt_softplus ? 1 : 0, dt_min, dt_max,
               init_state, y, final_state, static_cast<char *>(workspace), seq_idx,
               chunk_states};
    a.ev = kernel_events;
    // caller chunks shorter than the computed ones: the scan keeps the states
    // after its own chunks in the workspace, and the states the caller asked
    // for are stepped from those
    const bool fill = chunk_states && pl.Qs != pl.Q;
    float *Hc = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.off_hc);
    if (fill) a.states = Hc;
    hipError_t e = io_dtype == SSD_BF16 ? dispatch_scan<bf16>(pl, a, s)
                                        : dispatch_scan<float>(pl, a, s);
    if (e == hipSuccess && fill) {
        a.states = chunk_states;
        e = launch_token_states(pl, a, Hc, s);
    }
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

int32_t ssd_step(float *state, const void *x, const void *dt, const float *A, const void *B,
                 const void *C, const float *D, const float *dt_bias, int32_t dt_softplus,
                 float dt_min, float dt_max, void *y, int64_t batch, int64_t heads,
                 int64_t head_dim, int64_t state_dim, int64_t groups, int32_t io_dtype,
                 void *hip_stream) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0 || groups <= 0 ||
        heads % groups != 0)
        return SSD_ERR_SHAPE;
    if (!supported_dims(head_dim, state_dim)) return SSD_ERR_UNSUPPORTED;
    if (batch == 0) return SSD_OK;
    if (!mul_ok(batch, heads, (int64_t)1 << 40)) return SSD_ERR_UNSUPPORTED;
    if (!state || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    const size_t es = io_dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(state, 16) || !aligned(x, 4 * es) || !aligned(y, 4 * es) || !aligned(dt, es) ||
        !aligned(B, es) || !aligned(C, es) || !aligned(A, 4) || !aligned(D, 4) ||
        !aligned(dt_bias, 4))
        return SSD_ERR_ALIGN;
    StepArgs a{state, x, dt, B, C, A, D, dt_bias, dt_softplus ? 1 : 0, dt_min, dt_max, y,
               batch, heads, head_dim, state_dim, groups, io_dtype};
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = io_dtype == SSD_BF16 ? dispatch_step<bf16>(a, s) : dispatch_step<float>(a, s);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
