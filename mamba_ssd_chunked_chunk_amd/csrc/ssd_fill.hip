// States at the caller's chunk boundaries when the caller's chunk is shorter
// than the computed one (nnterp guide, "The state after every token": chunk
// size 1 makes every token a chunk boundary, so the states tensor holds the
// state after every token).
//
// The scan computes chunks of a whole number of caller chunks and keeps the
// fp32 state after each of them.  From the state entering a computed chunk
// (the initial state, or the state after the chunk before), this pass steps
// the Mamba-2 mixer's recurrence (nnterp guide, "Mamba-2" page: per head,
// with the state a state_dim x head_dim matrix)
//     S <- exp(A d_t) S + d_t B_t x_t^T     (S <- 0 first where a new
//                                             document starts)
// token by token through the chunk and writes S after every caller chunk.
//
// Writing the states (state_dim * head_dim fp32 each) is the whole cost, so
// the layout serves HBM writes: one workgroup per (batch, computed chunk,
// head, slice of up to 32 head_dim columns); a lane owns 4 consecutive
// columns of up to 4 state rows, and the lanes of one row write one 128-byte
// piece (64 bytes for head_dim 16) with 16-byte streaming stores.  The
// token's time step, decay, x and B are loaded one token ahead.
#include <hip/hip_runtime.h>

#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

namespace {

constexpr int kFillRows = 4;  // state rows per lane at most (state_dim <= 128)

// One token's inputs for a lane: time step, x columns, B at the lane's rows,
// and whether the token starts a new document.
struct TokIn {
    float dt;
    f32x4 x;
    float Bv[kFillRows];
    bool reset;
};

template <typename IO>
__device__ __forceinline__ void load_tok(TokIn &v, int64_t t, const IO *dp, const IO *xp,
                                         const IO *bp, const int32_t *sq, int64_t xs,
                                         int64_t bs, int dts, int r0, int RS, int n) {
    v.dt = to_f32(dp[t * dts]);
    v.x = ld4(xp + t * xs);
#pragma unroll
    for (int k = 0; k < kFillRows; ++k) {
        const int row = r0 + k * RS;
        v.Bv[k] = row < n ? to_f32(bp[t * bs + row]) : 0.f;
    }
    v.reset = sq != nullptr && t > 0 && sq[t] != sq[t - 1];
}

template <typename IO>
__global__ __launch_bounds__(256) void k_token_states(
    const IO *__restrict__ x, const IO *__restrict__ Bm, const IO *__restrict__ dt,
    const float *__restrict__ A, const float *__restrict__ dt_bias, int softplus, float dt_min,
    float dt_max, const int32_t *__restrict__ seq, const float *__restrict__ init,
    const float *__restrict__ Hc, float *__restrict__ out, int64_t l, int h, int g, int n,
    int p, int64_t Q, int64_t Qs, int64_t nc, int64_t ns) {
    const int PT = p < 32 ? p : 32;  // head_dim columns of the workgroup
    const int LR = PT / 4;           // lanes per state row
    const int RS = 256 / LR;         // rows per pass of the workgroup
    const int npt = p / PT;
    int64_t item = blockIdx.x;
    const int pt = (int)(item % npt);
    item /= npt;
    const int hh = (int)(item % h);
    item /= h;
    const int64_t c = item % nc;
    const int64_t b = item / nc;
    const int gi = hh / (h / g);
    const int tid = threadIdx.x, q = tid % LR, r0 = tid / LR;
    const int col = pt * PT + 4 * q;
    const int64_t np = (int64_t)n * p;

    // the state entering the computed chunk
    const float *src = c > 0 ? Hc + ((b * nc + c - 1) * h + hh) * np
                             : (init ? init + (b * h + hh) * np : nullptr);
    f32x4 H[kFillRows];
#pragma unroll
    for (int k = 0; k < kFillRows; ++k) {
        const int row = r0 + k * RS;
        H[k] = (src && row < n) ? *reinterpret_cast<const f32x4 *>(src + row * p + col)
                                : zero4();
    }
    const int64_t t0 = c * Q, t1 = (t0 + Q < l) ? t0 + Q : l;
    const float a2 = A[hh] * kLog2e;
    const float bias = dt_bias ? dt_bias[hh] : 0.f;
    const int64_t xs = (int64_t)h * p, bs = (int64_t)g * n;
    const IO *xp = x + (b * l * h + hh) * (int64_t)p + col;
    const IO *bp = Bm + (b * l * g + gi) * (int64_t)n;
    const IO *dp = dt + b * l * h + hh;
    const int32_t *sq = seq ? seq + b * l : nullptr;
    float *op = out + (b * ns * h + hh) * np + col;

    TokIn cur;
    load_tok(cur, t0, dp, xp, bp, sq, xs, bs, h, r0, RS, n);
    TokIn nxt = cur;
    for (int64_t t = t0; t < t1; ++t) {
        if (t + 1 < t1) load_tok(nxt, t + 1, dp, xp, bp, sq, xs, bs, h, r0, RS, n);
        const float d = time_step(cur.dt, bias, softplus, dt_min, dt_max);
        const float alpha = exp2_fast(a2 * d);
        const f32x4 dx = d * cur.x;
#pragma unroll
        for (int k = 0; k < kFillRows; ++k) {
            if (cur.reset) H[k] = zero4();
            H[k] = alpha * H[k] + cur.Bv[k] * dx;
        }
        if ((t + 1) % Qs == 0 || t == l - 1) {
            float *o = op + (t / Qs) * h * np;
#pragma unroll
            for (int k = 0; k < kFillRows; ++k) {
                const int row = r0 + k * RS;
                if (row < n)
                    __builtin_nontemporal_store(H[k],
                                                reinterpret_cast<f32x4 *>(o + (int64_t)row * p));
            }
        }
        cur = nxt;
    }
}

}  // namespace

hipError_t launch_token_states(const ScanPlan &pl, const ScanArgs &a, const float *Hc,
                               hipStream_t s) {
    const int64_t npt = pl.p < 32 ? 1 : pl.p / 32;
    const unsigned grid = (unsigned)(pl.b * pl.nc * pl.h * npt);
    if (pl.io == 1)
        return launch_timed(&k_token_states<bf16>, dim3(grid), dim3(256), s, a.ev, kSlotFill,
                            static_cast<const bf16 *>(a.x), static_cast<const bf16 *>(a.B),
                            static_cast<const bf16 *>(a.dt), a.A, a.dt_bias, a.softplus,
                            a.dt_min, a.dt_max, a.seq, a.init, Hc, a.states, pl.l, (int)pl.h,
                            (int)pl.g, (int)pl.n, (int)pl.p, pl.Q, pl.Qs, pl.nc, pl.ns);
    return launch_timed(&k_token_states<float>, dim3(grid), dim3(256), s, a.ev, kSlotFill,
                        static_cast<const float *>(a.x), static_cast<const float *>(a.B),
                        static_cast<const float *>(a.dt), a.A, a.dt_bias, a.softplus,
                        a.dt_min, a.dt_max, a.seq, a.init, Hc, a.states, pl.l, (int)pl.h,
                        (int)pl.g, (int)pl.n, (int)pl.p, pl.Q, pl.Qs, pl.nc, pl.ns);
}

}  // namespace ssd
