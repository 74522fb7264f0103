// Splitting one sequence into segments (one per GPU for long contexts):
// every segment is scanned from a zero state, which gives its own final
// state S_k; with its total log decay L_k (the sum of A d_t over its
// tokens), the state entering segment k follows from the earlier segments
// alone,
//     entry_0 = init,   entry_{k+1} = exp(L_k) entry_k + S_k,
// because the state after a stretch of tokens is a linear function of the
// state entering it (nnterp guide, "The state after every token": each
// boundary state is a cumulative function of the initial state; kongchang
// "Mamba2" page: the states pass serially from chunk to chunk).  Scanning
// segment k again from entry_k then gives its y and states exactly as one
// pass over the whole sequence would, up to rounding.
//
//   ssd_segment_log_decay  L per (batch, head) of one segment (-inf if a
//                          new document starts inside it)
//   ssd_combine_segments   the entry states of K segments, and the final
//                          state, from their (L_k, S_k) and the initial state
//
// Both are deterministic (fixed summation order).  Between GPUs the only
// exchange is the K pairs (L_k, S_k): state_dim * head_dim + 1 floats per
// (batch, head) and segment.
#include <hip/hip_runtime.h>

#include <math.h>

#include "../../include/ssd.h"
#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

namespace {

// One workgroup per (batch, head): the threads sum strided tokens in fp64,
// then a tree in LDS (fixed order).
template <typename IO>
__global__ __launch_bounds__(256) void k_segment_log_decay(
    const IO *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ dt_bias,
    int softplus, float dt_min, float dt_max, const int32_t *__restrict__ seq,
    float *__restrict__ out, int64_t l, int h) {
    __shared__ double red[256];
    __shared__ int cut[256];
    const int64_t pr = blockIdx.x, b = pr / h;
    const int hh = (int)(pr % h), tid = threadIdx.x;
    const float Ah = A[hh], bias = dt_bias ? dt_bias[hh] : 0.f;
    double s = 0.0;
    int c = 0;
    for (int64_t t = tid; t < l; t += 256) {
        const float d = time_step(to_f32(dt[(b * l + t) * h + hh]), bias, softplus, dt_min, dt_max);
        s += (double)Ah * (double)d;
        if (seq && t > 0 && seq[b * l + t] != seq[b * l + t - 1]) c = 1;
    }
    red[tid] = s;
    cut[tid] = c;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) {
            red[tid] += red[tid + off];
            cut[tid] |= cut[tid + off];
        }
        __syncthreads();
    }
    if (tid == 0) out[pr] = cut[0] ? -INFINITY : (float)red[0];
}

// One thread per state element: the K segments in order.
__global__ void k_combine_segments(const float *__restrict__ L, const float *__restrict__ S,
                                   const float *__restrict__ init,
                                   const int32_t *__restrict__ starts, float *__restrict__ entry,
                                   float *__restrict__ fin, int64_t K, int64_t b_, int64_t h,
                                   int64_t np) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = b_ * h * np;
    if (i >= total) return;
    const int64_t pr = i / np, b = pr / h;
    float cur = init ? init[i] : 0.f;
    for (int64_t k = 0; k < K; ++k) {
        // a segment whose first token starts a new document takes no state in
        if (starts && starts[k * b_ + b]) cur = 0.f;
        if (entry) entry[k * total + i] = cur;
        cur = expf(L[k * b_ * h + pr]) * cur + S[k * total + i];
    }
    if (fin) fin[i] = cur;
}

}  // namespace

}  // namespace ssd

using namespace ssd;

extern "C" {

int32_t ssd_segment_log_decay(const void *dt, const float *A, const float *dt_bias,
                              int32_t dt_softplus, float dt_min, float dt_max,
                              const int32_t *seq_idx, float *log_decay, int64_t batch,
                              int64_t seqlen, int64_t heads, int32_t io_dtype,
                              void *hip_stream) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || seqlen < 0 || heads <= 0) return SSD_ERR_SHAPE;
    if (batch * heads > ((int64_t)1 << 31) - 1) return SSD_ERR_UNSUPPORTED;
    if (batch == 0) return SSD_OK;
    if (!A || !log_decay || (seqlen > 0 && !dt)) return SSD_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const dim3 grid((unsigned)(batch * heads));
    if (io_dtype == SSD_BF16)
        hipLaunchKernelGGL((k_segment_log_decay<bf16>), grid, dim3(256), 0, s,
                           static_cast<const bf16 *>(dt), A, dt_bias, dt_softplus ? 1 : 0,
                           dt_min, dt_max, seq_idx, log_decay, seqlen, (int)heads);
    else
        hipLaunchKernelGGL((k_segment_log_decay<float>), grid, dim3(256), 0, s,
                           static_cast<const float *>(dt), A, dt_bias, dt_softplus ? 1 : 0,
                           dt_min, dt_max, seq_idx, log_decay, seqlen, (int)heads);
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

int32_t ssd_combine_segments(const float *log_decay, const float *seg_states,
                             const float *init_state, const int32_t *starts_document,
                             float *entry_states, float *final_state, int64_t segments,
                             int64_t batch, int64_t heads, int64_t head_dim, int64_t state_dim,
                             void *hip_stream) {
    if (segments <= 0 || batch < 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0)
        return SSD_ERR_SHAPE;
    if (batch == 0) return SSD_OK;
    if (!log_decay || !seg_states) return SSD_ERR_NULL;
    const int64_t total = batch * heads * head_dim * state_dim;
    if ((total + 255) / 256 > ((int64_t)1 << 31) - 1) return SSD_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipLaunchKernelGGL(k_combine_segments, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       s, log_decay, seg_states, init_state, starts_document, entry_states,
                       final_state, segments, batch, heads, head_dim * state_dim);
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
