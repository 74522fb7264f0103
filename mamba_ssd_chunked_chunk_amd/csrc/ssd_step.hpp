// One decode step of the SSD recurrence (nnterp guide, "Mamba-2" page,
// section "The state between steps": no sequence axis, the state is
// rewritten in place and only y is returned):
//     d = clamp(softplus(dt + dt_bias)),  alpha = exp(A d)
//     S[n][p] <- alpha S[n][p] + d B[n] x[p]
//     y[p]     = sum_n C[n] S[n][p] + D x[p]
//
// The state stream (state_dim * head_dim fp32, read once and written once)
// is the whole cost, so the kernel is laid out for HBM: one wave per
// (batch, head); each lane owns 4 consecutive head_dim columns, 64 lanes
// cover 256 / head_dim state rows per 16-byte vector access, every row is
// one fully used 64-byte-multiple segment, loads are issued in batches of
// RB rows per lane before any arithmetic, and the column sums of y are
// finished with cross-lane shuffles.  alpha and d are wave-uniform.
#pragma once

#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

template <typename IO, int P, int N>
__global__ __launch_bounds__(256) void k_step(
    float *__restrict__ state, const IO *__restrict__ x, const IO *__restrict__ dt,
    const float *__restrict__ A, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ dt_bias, int softplus, float dt_min,
    float dt_max, IO *__restrict__ y, int64_t pairs, int h, int g) {
    constexpr int LPR = P / 4;             // lanes per state row
    constexpr int RPI = 64 / LPR;          // rows per vector access of the wave
    constexpr int ITER = N / RPI;          // accesses per lane
    constexpr int RB = ITER < 16 ? ITER : 16;  // rows batched per lane
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * kWaves + wave;
    if (pair >= pairs) return;
    const int hh = (int)(pair % h);
    const int64_t b = pair / h;
    const int gi = hh / (h / g);
    const int q = lane % LPR, rsub = lane / LPR;

    const float d = time_step(to_f32(dt[pair]), dt_bias ? dt_bias[hh] : 0.f, softplus, dt_min,
                              dt_max);
    const float alpha = exp2_fast(A[hh] * d * kLog2e);
    const f32x4 xv = ld4(x + pair * P + q * 4);
    const f32x4 dx = d * xv;
    const IO *Bv = Bm + (b * g + gi) * N;
    const IO *Cv = Cm + (b * g + gi) * N;
    float *S = state + pair * (int64_t)N * P + q * 4;

    f32x4 yacc = zero4();
    for (int i0 = 0; i0 < ITER; i0 += RB) {
        f32x4 sv[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const int row = (i0 + k) * RPI + rsub;
            sv[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (int64_t)row * P));
        }
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const int row = (i0 + k) * RPI + rsub;
            const float bn = to_f32(Bv[row]), cn = to_f32(Cv[row]);
            const f32x4 nv = alpha * sv[k] + bn * dx;
            yacc += cn * nv;
            __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(S + (int64_t)row * P));
        }
    }
    // sum the RPI row groups: lanes q, q + LPR, q + 2 LPR, ...
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] += __shfl_xor(yacc[r], off, 64);
    }
    if (rsub == 0) {
        const float Dh = D ? D[hh] : 0.f;
        st4(y + pair * P + q * 4, yacc + Dh * xv);
    }
}

template <typename IO, int P, int N>
hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    const int64_t pairs = a.b * a.h;
    const unsigned nblk = (unsigned)((pairs + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((k_step<IO, P, N>), dim3(nblk), dim3(256), 0, s, a.state,
                       static_cast<const IO *>(a.x), static_cast<const IO *>(a.dt), a.A,
                       static_cast<const IO *>(a.B), static_cast<const IO *>(a.C), a.D, a.dt_bias,
                       a.softplus, a.dt_min, a.dt_max, static_cast<IO *>(a.y), pairs, (int)a.h,
                       (int)a.g);
    return hipGetLastError();
}

}  // namespace ssd
