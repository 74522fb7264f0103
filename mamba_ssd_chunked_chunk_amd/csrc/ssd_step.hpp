// One decode step of the SSD recurrence (nnterp guide, "Mamba-2" page,
// section "The state between steps": no sequence axis, the state is
// rewritten in place and only y is returned):
//     d = clamp(softplus(dt + dt_bias)),  alpha = exp(A d)
//     S[n][p] <- alpha S[n][p] + d B[n] x[p]
//     y[p]     = sum_n C[n] S[n][p] + D x[p]
//
// The state stream (state_dim * head_dim fp32, read once and written once)
// is the whole cost, so the kernel is laid out for HBM: one wave per
// (batch, head); each lane owns 4 consecutive head_dim columns of a run of
// consecutive state rows (64 lanes: 256 / head_dim runs of state_dim *
// head_dim / 256 rows), so every wave access is 256 / head_dim fully used
// segments of head_dim fp32.  The lane's first RB state rows are requested
// before anything else (they need nothing computed), then the time step, x
// and the lane's run of B and C (a few 16-byte loads); no branch merges a
// loaded value, so all of it is in flight together.  (The first version
// waited for the time step and x before requesting any state row and read
// B and C one element per row: 236 us against 217 us at the decode
// workload.)  The column sums of y
// are finished with cross-lane shuffles; alpha and d are wave-uniform.
#pragma once

#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

// The M consecutive io values at p as loaded: 16 bytes at a time where VEC
// (p 16-byte aligned) and M * sizeof(IO) is a multiple of 16, else element
// by element.
template <typename IO, int M, bool VEC> struct Run {
    static constexpr bool R16 = VEC && (M * sizeof(IO)) % 16 == 0;
    static constexpr int NV = R16 ? M * sizeof(IO) / 16 : 1;
    u32x4 v[NV];
    IO e[R16 ? 1 : M];
    __device__ __forceinline__ void load(const IO *p) {
        if constexpr (R16) {
#pragma unroll
            for (int i = 0; i < NV; ++i) v[i] = reinterpret_cast<const u32x4 *>(p)[i];
        } else {
#pragma unroll
            for (int i = 0; i < M; ++i) e[i] = p[i];
        }
    }
    __device__ __forceinline__ float at(int i) const {
        if constexpr (R16) {
            const IO *q = reinterpret_cast<const IO *>(&v[0]);
            return to_f32(q[i]);
        } else {
            return to_f32(e[i]);
        }
    }
};

// VB: B and C 16-byte aligned (their runs then load 16 bytes at a time)
template <typename IO, int P, int N, bool VB>
__global__ __launch_bounds__(256) void k_step(
    float *__restrict__ state, const IO *__restrict__ x, const IO *__restrict__ dt,
    const float *__restrict__ A, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ dt_bias, int softplus, float dt_min,
    float dt_max, IO *__restrict__ y, int64_t pairs, int h, int g) {
    constexpr int LPR = P / 4;                 // lanes per state row
    constexpr int RPI = 64 / LPR;              // row runs per wave
    constexpr int ITER = N / RPI;              // rows per run (one access each)
    // rows in flight per lane: 16 (decode workload, 256 x 80 heads: 216.5 us
    // against 218.5 with 8 and 234 with 32, whose 211 registers leave two
    // waves per SIMD)
    constexpr int RB = ITER < 16 ? ITER : 16;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * kWaves + wave;
    if (pair >= pairs) return;
    const int hh = (int)(pair % h);
    const int64_t b = pair / h;
    const int gi = hh / (h / g);
    const int q = lane % LPR, rsub = lane / LPR;
    const int r0 = rsub * ITER;  // the lane's rows r0 .. r0 + ITER - 1
    float *S = state + pair * (int64_t)N * P + (int64_t)r0 * P + q * 4;

    f32x4 sv[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k)
        sv[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (int64_t)k * P));
    const IO dtr = dt[pair];
    const f32x4 xv = ld4(x + pair * P + q * 4);
    Run<IO, ITER, VB> Br, Cr;
    Br.load(Bm + (b * g + gi) * N + r0);
    Cr.load(Cm + (b * g + gi) * N + r0);
    const float Ah = A[hh];
    const float bias = dt_bias ? dt_bias[hh] : 0.f;
    const float Dh = D ? D[hh] : 0.f;

    const float d = time_step(to_f32(dtr), bias, softplus, dt_min, dt_max);
    const float alpha = exp2_fast(Ah * d * kLog2e);
    const f32x4 dx = d * xv;
    f32x4 yacc = zero4();
#pragma unroll
    for (int i0 = 0; i0 < ITER; i0 += RB) {
        if (i0 > 0) {
#pragma unroll
            for (int k = 0; k < RB; ++k)
                sv[k] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4 *>(S + (int64_t)(i0 + k) * P));
        }
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const float bn = Br.at(i0 + k), cn = Cr.at(i0 + k);
            const f32x4 nv = alpha * sv[k] + bn * dx;
            yacc += cn * nv;
            __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(S + (int64_t)(i0 + k) * P));
        }
    }
    // sum the RPI row runs: lanes q, q + LPR, q + 2 LPR, ...
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] += __shfl_xor(yacc[r], off, 64);
    }
    if (rsub == 0) st4(y + pair * P + q * 4, yacc + Dh * xv);
}

template <typename IO, int P, int N>
hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    const int64_t pairs = a.b * a.h;
    const unsigned nblk = (unsigned)((pairs + kWaves - 1) / kWaves);
    const bool vb = ((uintptr_t)a.B & 15) == 0 && ((uintptr_t)a.C & 15) == 0;
    auto go = [&](auto vb_c) {
        hipLaunchKernelGGL((k_step<IO, P, N, decltype(vb_c)::value>), dim3(nblk), dim3(256), 0,
                           s, a.state, static_cast<const IO *>(a.x),
                           static_cast<const IO *>(a.dt), a.A, static_cast<const IO *>(a.B),
                           static_cast<const IO *>(a.C), a.D, a.dt_bias, a.softplus, a.dt_min,
                           a.dt_max, static_cast<IO *>(a.y), pairs, (int)a.h, (int)a.g);
    };
    if (vb) go(std::true_type{});
    else go(std::false_type{});
    return hipGetLastError();
}

}  // namespace ssd
