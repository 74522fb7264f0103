// Gradient pass of the chunked scan, deterministic (every sum in a fixed
// order, no atomics).
//
// The forward is the per-head recurrence of the nnterp guide's "Mamba-2"
// page: h_t = alpha_t h_{t-1} + d_t B_t x_t^T, y_t = C_t^T h_t + D x_t, with
// alpha_t = exp(A d_t).  Its adjoint state g_t = dL/dh_t obeys the same
// kind of recurrence backwards in time,
//     g_t = alpha_{t+1} g_{t+1} + C_t dy_t^T,
// so the gradients come from three runs of the fp32 chunked scan on
// rearranged operands (t' = l - 1 - t reverses time):
//   1. the adjoint:  state g (n x p), inputs C (as B) and dy (as x), weight
//      1, decay alpha_{t+1}, reversed; its read-out with B gives
//      yb_t = g_t^T B_t, hence dx_t = D dy_t + d_t yb_t, and its final state
//      g_0 gives d init = alpha_0 g_0;
//   2. the forward transposed:  state h^T (p x n), inputs x (as B, one group
//      per head) and B (as x), the forward's own time steps; its read-out
//      with dy gives h_t dy_t, every head's part of dC_t; its final state is
//      h_l^T;
//   3. the adjoint transposed:  state g^T, inputs dy (as B) and C (as x),
//      reversed; its read-out with x gives g_t x_t, every head's part of
//      dB_t / d_t.
// The log-decay gradient da_t = alpha_t <g_t, h_{t-1}> needs no state: with
// u_t = dy_t . (C_t^T h_t) and v_t = d_t yb_t . x_t, the identity
// <g_t, h_t> = u_t + <g_{t+1}, h_{t+1}> - v_{t+1} (inside a document) makes
// da_t a reverse running sum of u - v (plus <d_final, h_l> in the last
// document), taken per (batch, head) in fp64.  Then dd_t = yb_t . x_t +
// A da_t, ddt through the clamp and softplus, dA = sum d da, and the sums
// over the group's heads and over the batch in fixed order.
#include <hip/hip_runtime.h>

#include <math.h>

#include "../../include/ssd.h"
#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

namespace {

// fp32 workspace of the gradient pass (offsets in bytes)
struct BwdPlan {
    ScanPlan s1, s2;  // the adjoint scan (p, n, g); the transposed scans (n, p, h groups)
    size_t dyR, xR, xF, dyF, CR, BR, Bh, CRh, dtF, lw, la, seqR, y1, y2, y3, sc, part, term,
        fin1, finT, initT, dfT, ws, total;
};

bool make_bwd_plan(BwdPlan &P, int64_t b, int64_t l, int64_t h, int64_t p, int64_t n,
                   int64_t g, int64_t Q) {
    if (!make_plan(P.s1, b, l, h, p, n, g, Q, 0)) return false;
    if (!make_plan(P.s2, b, l, h, n, p, h, Q, 0)) return false;
    const int64_t thp = b * l * h * p * 4, tgn = b * l * g * n * 4, thn = b * l * h * n * 4;
    const int64_t th = b * l * h * 4, st = b * h * n * p * 4;
    size_t o = 0;
    auto take = [&](size_t &off, int64_t bytes) { off = o; o += align256(bytes); };
    take(P.dyR, thp); take(P.xR, thp); take(P.xF, thp); take(P.dyF, thp);
    take(P.CR, tgn); take(P.BR, tgn); take(P.Bh, thn); take(P.CRh, thn);
    take(P.dtF, th); take(P.lw, th); take(P.la, th); take(P.seqR, b * l * 4);
    take(P.y1, thp); take(P.y2, thn); take(P.y3, thn);
    take(P.sc, th * 4); take(P.part, b * h * 3 * 8); take(P.term, b * h * 8);
    take(P.fin1, st); take(P.finT, st); take(P.initT, st); take(P.dfT, st);
    take(P.ws, (int64_t)(P.s1.total > P.s2.total ? P.s1.total : P.s2.total));
    P.total = o;
    return true;
}

// Workspace of the bf16 gradient pass: reversed bf16 copies of the inputs
// the two adjoint scans read, the scans' fp32 outputs and the shared tail.
struct BwdPlan16 {
    ScanPlan s1, s2;
    size_t y1, y2, y3, du, dw, sc, part, term, fin1, finT, initT, dfT, ws, total;
    int nparts;  // waves per head of the transposed scans (their row-dot parts)
};

// The parts of a scan plan's workspace the bf16 kernels use (scaled fp16
// boundary and chunk states, per-chunk decays, maxima and scales), packed
// from offset 0; the fp32 path's per-row arrays and fp32-sized states are
// left out.
void compact_bf16(ScanPlan &pl) {
    const int64_t sts = pl.b * pl.nc * pl.h * pl.n * pl.p * 2, per = pl.b * pl.h * pl.nc * 4;
    size_t o = 0;
    auto take = [&](size_t &off, int64_t bytes) { off = o; o += align256(bytes); };
    take(pl.off_hb, sts); take(pl.off_st, sts); take(pl.off_lam, per); take(pl.off_scl, per);
    take(pl.off_hs, per); take(pl.off_imx, pl.b * pl.h * 4);
    pl.off_lcs = pl.off_dtp = pl.off_wgt = pl.off_sgr = pl.off_img = pl.off_hc = o;
    pl.total = o;
}

bool make_bwd_plan16(BwdPlan16 &P, int64_t b, int64_t l, int64_t h, int64_t p, int64_t n,
                     int64_t g, int64_t Q) {
    if (!make_plan(P.s1, b, l, h, p, n, g, Q, 1)) return false;
    if (!make_plan(P.s2, b, l, h, n, p, h, Q, 1)) return false;
    compact_bf16(P.s1);
    compact_bf16(P.s2);
    const int64_t thp = b * l * h * p, thn = b * l * h * n;
    const int64_t th = b * l * h, st = b * h * n * p * 4;
    size_t o = 0;
    auto take = [&](size_t &off, int64_t bytes) { off = o; o += align256(bytes); };
    P.nparts = n >= 128 ? (int)(n / 64) : 1;
    take(P.y1, thp * 2); take(P.y2, thn * 2); take(P.y3, thn * 2);
    take(P.du, th * P.nparts * 4); take(P.dw, th * P.nparts * 4);
    take(P.sc, th * 16); take(P.part, b * h * 3 * 8); take(P.term, b * h * 8);
    take(P.fin1, st); take(P.finT, st); take(P.initT, st); take(P.dfT, st);
    take(P.ws, (int64_t)(P.s1.total > P.s2.total ? P.s1.total : P.s2.total));
    P.total = o;
    return true;
}

struct BwdBufs {
    float *dyR, *xR, *xF, *dyF, *CR, *BR, *Bh, *CRh, *dtF, *lw, *la, *y1, *y2, *y3, *sc;
    int32_t *seqR;
    double *part, *term;
    float *fin1, *finT, *initT, *dfT;
};

// The rearranged operands of the three scans, one workgroup per token.
template <typename IO>
__global__ __launch_bounds__(256) void k_bwd_prep(
    const IO *__restrict__ x, const IO *__restrict__ dt, const float *__restrict__ A,
    const IO *__restrict__ Bm, const IO *__restrict__ Cm, const IO *__restrict__ dy,
    const float *__restrict__ dt_bias, int softplus, float dt_min, float dt_max,
    const int32_t *__restrict__ seq, BwdBufs w, int64_t l, int h, int g, int p, int n) {
    const int64_t bt = blockIdx.x, b = bt / l, t = bt % l;
    const int64_t rt = b * l + (l - 1 - t);  // the reversed token's row
    const int tid = threadIdx.x;
    const int hp = h * p, gn = g * n, hn = h * n, hpg = h / g;
    for (int i = tid; i < hp; i += 256) {
        const float dv = to_f32(dy[bt * hp + i]), xv = to_f32(x[bt * hp + i]);
        w.dyR[rt * hp + i] = dv;
        w.xR[rt * hp + i] = xv;
        w.dyF[bt * hp + i] = dv;
        w.xF[bt * hp + i] = xv;
    }
    for (int i = tid; i < gn; i += 256) {
        w.CR[rt * gn + i] = to_f32(Cm[bt * gn + i]);
        w.BR[rt * gn + i] = to_f32(Bm[bt * gn + i]);
    }
    for (int i = tid; i < hn; i += 256) {
        const int hh = i / n, k = i % n;
        const int64_t src = bt * gn + (hh / hpg) * n + k;
        w.Bh[bt * hn + i] = to_f32(Bm[src]);
        w.CRh[rt * hn + i] = to_f32(Cm[src]);
    }
    for (int i = tid; i < h; i += 256) {
        w.dtF[bt * h + i] = to_f32(dt[bt * h + i]);
        w.lw[rt * h + i] = 1.f;
        // the reversed step t' carries the decay of forward token t + 1
        float la = 0.f;
        if (t + 1 < l) {
            const float d1 = time_step(to_f32(dt[(bt + 1) * h + i]), dt_bias ? dt_bias[i] : 0.f,
                                       softplus, dt_min, dt_max);
            la = A[i] * d1 * kLog2e;
        }
        w.la[rt * h + i] = la;
    }
    if (seq && tid == 0) w.seqR[rt] = seq[bt];
}

// The two bf16 values of a 32-bit word as fp32 (exact), and two fp32
// values rounded to bf16 (nearest even) as one word.
__device__ __forceinline__ float bf16_bits_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_bits_hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16 ha = (bf16)a, hb = (bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// [pairs][n][p] -> [pairs][p][n], element by element (the fp32 pass)
__global__ void k_transpose_np(const float *__restrict__ src, float *__restrict__ dst,
                               int64_t pairs, int n, int p) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t np = (int64_t)n * p;
    if (i >= pairs * np) return;
    const int64_t pr = i / np, r = i % np, k = r / p, j = r % p;
    dst[pr * np + j * n + k] = src[i];
}

// The same through 32 x 32 tiles in LDS, reads and writes along rows: one
// workgroup (32 x 8 threads) per tile of one pair; n and p are multiples of
// 32.
__global__ __launch_bounds__(256) void k_transpose_tiles(const float *__restrict__ src,
                                                         float *__restrict__ dst, int n, int p) {
    __shared__ float tile[32][33];
    const int64_t pr = blockIdx.z;
    const int k0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const float *s0 = src + pr * (int64_t)n * p;
    float *d0 = dst + pr * (int64_t)n * p;
#pragma unroll
    for (int r = ty; r < 32; r += 8) tile[r][tx] = s0[(int64_t)(k0 + r) * p + j0 + tx];
    __syncthreads();
#pragma unroll
    for (int r = ty; r < 32; r += 8) d0[(int64_t)(j0 + r) * n + k0 + tx] = tile[tx][r];
}

// Per token and head (16 lanes, 4 consecutive elements each): dx, and the
// scalars u - v, yb . x, dy . x and d for the running sums.
template <typename IO>
__global__ __launch_bounds__(256) void k_bwd_tok(
    const IO *__restrict__ x, const IO *__restrict__ dt, const IO *__restrict__ Cm,
    const IO *__restrict__ dy, const float *__restrict__ D, const float *__restrict__ dt_bias,
    int softplus, float dt_min, float dt_max, BwdBufs w, IO *__restrict__ dx, int64_t bl,
    int64_t l, int h, int g, int p, int n) {
    const int lane = threadIdx.x & 63, sl = lane & 15;
    const int64_t item0 = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool valid = item0 < bl * h;
    const int64_t item = valid ? item0 : 0;  // every lane takes part in the shuffles
    const int64_t bt = item / h, b = bt / l, t = bt % l;
    const int hh = (int)(item % h), gi = hh / (h / g);
    const int64_t rt = b * l + (l - 1 - t);
    const float d = time_step(to_f32(dt[bt * h + hh]), dt_bias ? dt_bias[hh] : 0.f, softplus,
                              dt_min, dt_max);
    const float Dh = D ? D[hh] : 0.f;
    float wsum = 0.f, dsum = 0.f, usum = 0.f;
    for (int j = sl * 4; j < p; j += 64) {
        const int64_t at = (bt * h + hh) * p + j;
        const f32x4 yb = *reinterpret_cast<const f32x4 *>(w.y1 + (rt * h + hh) * p + j);
        const f32x4 xv = ld4(x + at), dv = ld4(dy + at);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wsum += yb[e] * xv[e];
            dsum += dv[e] * xv[e];
        }
        if (valid) st4(dx + at, Dh * dv + d * yb);
    }
    for (int k = sl * 4; k < n; k += 64) {
        const f32x4 cv = ld4(Cm + (bt * g + gi) * n + k);
        const f32x4 yv = *reinterpret_cast<const f32x4 *>(w.y2 + (bt * h + hh) * n + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) usum += cv[e] * yv[e];
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
        wsum += __shfl_xor(wsum, off, 64);
        dsum += __shfl_xor(dsum, off, 64);
        usum += __shfl_xor(usum, off, 64);
    }
    if (valid && sl == 0) {
        float *o = w.sc + ((b * h + hh) * l + t) * 4;
        *reinterpret_cast<f32x4 *>(o) = f32x4{usum - d * wsum, wsum, dsum, d};
    }
}

// The bf16 pass's per-token step, one workgroup per token: per head (16
// lanes, 4 consecutive elements each) dx = D dy + d yb, and the scalars
// u - v, yb . x, dy . x and d for the running sums, with u = C . (h dy) and
// yb . x = B . (g x) summed from the transposed scans' row dots (fp32, one
// part per wave); then dB and dC, the group's heads summed in a fixed order
// from the bf16 read-outs.  The heads' d are kept in LDS for the second
// step (up to kTokHeads heads; beyond, taken from the time steps again).
constexpr int kTokHeads = 1024;

__global__ __launch_bounds__(256) void k_bwd_tokg(
    const bf16 *__restrict__ x, const bf16 *__restrict__ dt, const bf16 *__restrict__ dy,
    const float *__restrict__ D, const float *__restrict__ dt_bias, int softplus, float dt_min,
    float dt_max, const bf16 *__restrict__ yb1, const bf16 *__restrict__ y2,
    const bf16 *__restrict__ y3, const float *__restrict__ du, const float *__restrict__ dw,
    int nparts, float *__restrict__ sc_out, bf16 *__restrict__ dx, bf16 *__restrict__ dB,
    bf16 *__restrict__ dC, int64_t l, int h, int g, int p, int n) {
    __shared__ float dsh[kTokHeads];
    const int64_t bt = blockIdx.x, b = bt / l, t = bt % l;
    const int tid = threadIdx.x;
    // p / 8 lanes per head, 8 elements each (16-byte rows); the lane groups
    // are whole and aligned in every round (256 threads)
    const int lph = p / 8, sl = tid & (lph - 1);
    for (int task = tid; task < h * lph; task += 256) {
        const int hh = task / lph;
        const float d = time_step(to_f32(dt[bt * h + hh]), dt_bias ? dt_bias[hh] : 0.f,
                                  softplus, dt_min, dt_max);
        const float Dh = D ? D[hh] : 0.f;
        const int64_t at = (bt * h + hh) * p + 8 * sl;
        const u32x4 yq = *reinterpret_cast<const u32x4 *>(yb1 + at);
        const u32x4 xq = *reinterpret_cast<const u32x4 *>(x + at);
        const u32x4 dq = *reinterpret_cast<const u32x4 *>(dy + at);
        float dsum = 0.f;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float d0 = bf16_bits_lo(dq[e]), d1 = bf16_bits_hi(dq[e]);
            dsum += d0 * bf16_bits_lo(xq[e]) + d1 * bf16_bits_hi(xq[e]);
            const float o0 = Dh * d0 + d * bf16_bits_lo(yq[e]);
            const float o1 = Dh * d1 + d * bf16_bits_hi(yq[e]);
            o[e] = pack_bf16x2(o0, o1);
        }
        *reinterpret_cast<u32x4 *>(dx + at) = o;
        for (int off = lph >> 1; off > 0; off >>= 1) dsum += __shfl_xor(dsum, off, 64);
        if (sl == 0) {
            float usum = 0.f, wsum = 0.f;
            for (int q = 0; q < nparts; ++q) {
                usum += du[(bt * h + hh) * nparts + q];
                wsum += dw[(bt * h + hh) * nparts + q];
            }
            float *o = sc_out + ((b * h + hh) * l + t) * 4;
            *reinterpret_cast<f32x4 *>(o) = f32x4{usum - d * wsum, wsum, dsum, d};
            if (hh < kTokHeads) dsh[hh] = d;
        }
    }
    __syncthreads();
    // dB, dC: 16 head sets (set j: heads j, j + 16, .. of the group, in
    // order) x n / 8 lanes of 8 consecutive elements; the sets' partial
    // sums are added in set order through LDS
    __shared__ f32x4 pb[16][16][2], pc[16][16][2];
    const int hpg = h / g, kl = tid & 15, js = tid >> 4, nk = n / 8;
    for (int gi = 0; gi < g; ++gi) {
        f32x4 sb0 = zero4(), sb1 = zero4(), sc0 = zero4(), sc1 = zero4();
        if (kl < nk) {
            for (int q = js; q < hpg; q += 16) {
                const int hh = gi * hpg + q;
                const float d = hh < kTokHeads
                                    ? dsh[hh]
                                    : time_step(to_f32(dt[bt * h + hh]),
                                                dt_bias ? dt_bias[hh] : 0.f, softplus, dt_min,
                                                dt_max);
                const u32x4 bq = *reinterpret_cast<const u32x4 *>(y3 + (bt * h + hh) * n + 8 * kl);
                const u32x4 cq = *reinterpret_cast<const u32x4 *>(y2 + (bt * h + hh) * n + 8 * kl);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    sb0[2 * e] += d * bf16_bits_lo(bq[e]);
                    sb0[2 * e + 1] += d * bf16_bits_hi(bq[e]);
                    sb1[2 * e] += d * bf16_bits_lo(bq[2 + e]);
                    sb1[2 * e + 1] += d * bf16_bits_hi(bq[2 + e]);
                    sc0[2 * e] += bf16_bits_lo(cq[e]);
                    sc0[2 * e + 1] += bf16_bits_hi(cq[e]);
                    sc1[2 * e] += bf16_bits_lo(cq[2 + e]);
                    sc1[2 * e + 1] += bf16_bits_hi(cq[2 + e]);
                }
            }
        }
        pb[js][kl][0] = sb0;
        pb[js][kl][1] = sb1;
        pc[js][kl][0] = sc0;
        pc[js][kl][1] = sc1;
        __syncthreads();
        if (js < 2 && kl < nk) {
            // thread (js, kl) finishes half js of lane kl's 8 elements
            f32x4 tb = zero4(), tc = zero4();
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                tb += pb[j][kl][js];
                tc += pc[j][kl][js];
            }
            st4(dB + (bt * g + gi) * n + 8 * kl + 4 * js, tb);
            st4(dC + (bt * g + gi) * n + 8 * kl + 4 * js, tc);
        }
        __syncthreads();
    }
}

// <d_final, h_l> per (batch, head), h_l^T from the transposed forward scan.
__global__ __launch_bounds__(256) void k_bwd_term(const float *__restrict__ dfin,
                                                  const float *__restrict__ finT,
                                                  double *__restrict__ term, int n, int p) {
    __shared__ double red[256];
    const int64_t pr = blockIdx.x;
    const int64_t np = (int64_t)n * p;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < np; i += 256) {
        const int64_t k = i / p, j = i % p;
        s += (double)dfin[pr * np + i] * (double)finT[pr * np + j * n + k];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) term[pr] = red[0];
}

// Per (batch, head), one workgroup: the reverse running sum of u - v
// (restarting where a document ends; the final-state term enters at the
// last token) gives da_t; then ddt and the (batch, head) parts of dA,
// d dt_bias and dD, all in fp64.  Thread k owns a contiguous segment of
// tokens; a segment acts on the sum entering it from the right as either
// "add S" or, with a document end inside, "restart at S"; thread 0 chains
// the segments right to left, then every thread walks its own tokens with
// the sum entering it.  Fixed order throughout.
constexpr int kCumThreads = 256;

template <typename IO>
__global__ __launch_bounds__(kCumThreads) void k_bwd_cum(
    const IO *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ dt_bias,
    int softplus, float dt_min, float dt_max, const int32_t *__restrict__ seq, int has_init,
    BwdBufs w, IO *__restrict__ ddt, int64_t l, int h, const float *__restrict__ tdf = nullptr,
    const float *__restrict__ tfin = nullptr, int64_t np = 0) {
    __shared__ double seg_val[kCumThreads], red[3][kCumThreads];
    __shared__ int seg_cut[kCumThreads];
    const int64_t pr = blockIdx.x;
    // with tdf: the final-state term <d_final, h_l> of this (batch, head)
    // from both in the same element order, summed here in fixed order
    double term = 0.0;
    if (tdf) {
        double s = 0.0;
        for (int64_t i = threadIdx.x; i < np; i += kCumThreads)
            s += (double)tdf[pr * np + i] * (double)tfin[pr * np + i];
        red[0][threadIdx.x] = s;
        __syncthreads();
        for (int off = kCumThreads / 2; off > 0; off >>= 1) {
            if ((int)threadIdx.x < off) red[0][threadIdx.x] += red[0][threadIdx.x + off];
            __syncthreads();
        }
        term = red[0][0];
        __syncthreads();
    } else if (w.term) {
        term = w.term[pr];
    }
    const int64_t b = pr / h;
    const int hh = (int)(pr % h), tid = threadIdx.x;
    const float Ah = A[hh], bias = dt_bias ? dt_bias[hh] : 0.f;
    const float *sc = w.sc + pr * l * 4;
    const int32_t *sq = seq ? seq + b * l : nullptr;
    const int64_t per = (l + kCumThreads - 1) / kCumThreads;
    const int64_t t0 = tid * per, t1 = (t0 + per < l) ? t0 + per : l;
    // does a document end after token t (before t + 1)?
    auto ends = [&](int64_t t) { return sq && t + 1 < l && sq[t + 1] != sq[t]; };
    // this segment's action on the sum entering it
    double acc = 0.0;
    int cut = 0;
    for (int64_t t = t1 - 1; t >= t0; --t) {
        if (ends(t)) {
            acc = 0.0;
            cut = 1;
        }
        acc += (double)sc[t * 4];
    }
    seg_val[tid] = acc;
    seg_cut[tid] = cut;
    __syncthreads();
    if (tid == 0) {
        // the sum entering each segment from the right, stored in seg_val
        double carry = term;
        for (int k = kCumThreads - 1; k >= 0; --k) {
            const double v = seg_val[k];
            const int c = seg_cut[k];
            seg_val[k] = carry;
            carry = c ? v : carry + v;
        }
    }
    __syncthreads();
    acc = seg_val[tid];
    double sA = 0.0, sB = 0.0, sD = 0.0;
    for (int64_t t = t1 - 1; t >= t0; --t) {
        if (ends(t)) acc = 0.0;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(sc + t * 4);
        acc += (double)v[0];
        double da = acc;
        // no state before a document's first token (or before token 0
        // without an initial state): no decay acts there
        if ((sq && t > 0 && sq[t] != sq[t - 1]) || (t == 0 && !has_init)) da = 0.0;
        const double dd = (double)v[1] + (double)Ah * da;
        const float z = to_f32(dt[(b * l + t) * h + hh]) + bias;
        const float spv = softplus ? (z > 20.f ? z : log1pf(expf(z))) : z;
        const bool pass = spv >= dt_min && spv <= dt_max;
        const double dsp = softplus ? (double)(1.f / (1.f + expf(-z))) : 1.0;
        const double g = pass ? dd * dsp : 0.0;
        ddt[(b * l + t) * h + hh] = (IO)(float)g;
        sA += (double)v[3] * da;
        sB += g;
        sD += (double)v[2];
    }
    red[0][tid] = sA;
    red[1][tid] = sB;
    red[2][tid] = sD;
    __syncthreads();
    for (int off = kCumThreads / 2; off > 0; off >>= 1) {
        if (tid < off)
#pragma unroll
            for (int q = 0; q < 3; ++q) red[q][tid] += red[q][tid + off];
        __syncthreads();
    }
    if (tid < 3) w.part[pr * 3 + tid] = red[tid][0];
}

// dB and dC of one token: the group's heads summed in order.
template <typename IO>
__global__ __launch_bounds__(256) void k_bwd_group(BwdBufs w, IO *__restrict__ dB,
                                                   IO *__restrict__ dC, int64_t l, int h, int g,
                                                   int n) {
    const int64_t bt = blockIdx.x, b = bt / l, t = bt % l;
    const int64_t rt = b * l + (l - 1 - t);
    const int hpg = h / g;
    for (int i = threadIdx.x; i < g * n; i += 256) {
        const int gi = i / n, k = i % n;
        float sb = 0.f, sc = 0.f;
        for (int q = 0; q < hpg; ++q) {
            const int hh = gi * hpg + q;
            const float d = w.sc[((b * h + hh) * l + t) * 4 + 3];
            sb += d * w.y3[(rt * h + hh) * n + k];
            sc += w.y2[(bt * h + hh) * n + k];
        }
        dB[bt * g * n + i] = (IO)sb;
        dC[bt * g * n + i] = (IO)sc;
    }
}

// dA, d dt_bias, dD: the (batch, head) parts summed over the batch in order.
__global__ void k_bwd_sum(const double *__restrict__ part, float *__restrict__ dA,
                          float *__restrict__ dbias, float *__restrict__ dD, int64_t b_, int h) {
    const int hh = blockIdx.x * blockDim.x + threadIdx.x;
    if (hh >= h) return;
    double a = 0.0, bi = 0.0, d = 0.0;
    for (int64_t b = 0; b < b_; ++b) {
        a += part[(b * h + hh) * 3 + 0];
        bi += part[(b * h + hh) * 3 + 1];
        d += part[(b * h + hh) * 3 + 2];
    }
    dA[hh] = (float)a;
    if (dbias) dbias[hh] = (float)bi;
    if (dD) dD[hh] = (float)d;
}

// d init = alpha_0 g_0.
__global__ void k_bwd_init(const float *__restrict__ fin1, const float *__restrict__ sc,
                           const float *__restrict__ A, float *__restrict__ dinit, int64_t pairs,
                           int h, int64_t l, int64_t np) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= pairs * np) return;
    const int64_t pr = i / np;
    const float d0 = sc[pr * l * 4 + 3];
    dinit[i] = expf(A[pr % h] * d0) * fin1[i];
}

bool al16(const void *q) { return ((uintptr_t)q & 15) == 0; }

// The gradient pass for bf16 io: the three scans on the bf16 kernels (bf16
// operands exact, derived operands as two bf16 terms, fp32 accumulation and
// fp32 outputs), the adjoint ones on reversed copies with unit weights and
// the next token's decay, the transposed ones reading the group's B or C
// rows for every head (x slot = head / heads per group) instead of
// broadcast copies; then the same per-token, running-sum and group-sum
// kernels as the fp32 pass.
int32_t bwd_bf16(const bf16 *x, const bf16 *dt, const float *A, const bf16 *B, const bf16 *C,
                 const float *D, const float *dt_bias, int32_t dt_softplus, float dt_min,
                 float dt_max, const float *init_state, const int32_t *seq_idx, const bf16 *dy,
                 const float *d_final, bf16 *dx, bf16 *ddt, float *dA, bf16 *dB, bf16 *dC,
                 float *dD, float *d_dt_bias, float *d_init, int64_t b, int64_t l, int64_t h,
                 int64_t p, int64_t n, int64_t g, int64_t chunk, void *workspace,
                 size_t workspace_bytes, hipStream_t s) {
    BwdPlan16 P;
    if (!make_bwd_plan16(P, b, l, h, p, n, g, chunk)) return SSD_ERR_SHAPE;
    const int64_t lim32 = (int64_t)1 << 31;
    if (P.s1.lp * 4 >= lim32 || P.s2.lp * 4 >= lim32) return SSD_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < P.total) return SSD_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    BwdBufs w{};
    w.sc = reinterpret_cast<float *>(ws + P.sc);
    w.part = reinterpret_cast<double *>(ws + P.part);
    w.term = d_final ? reinterpret_cast<double *>(ws + P.term) : nullptr;
    w.fin1 = reinterpret_cast<float *>(ws + P.fin1);
    w.finT = reinterpret_cast<float *>(ws + P.finT);
    w.initT = reinterpret_cast<float *>(ws + P.initT);
    w.dfT = reinterpret_cast<float *>(ws + P.dfT);
    char *scan_ws = ws + P.ws;
    const int64_t bl = b * l, pairs = b * h, np = n * p;
    const unsigned eblk = (unsigned)((pairs * np + 255) / 256);
    const int sp = dt_softplus ? 1 : 0;
    hipError_t e = hipSuccess;
    auto ok = [&]() { return (e = hipGetLastError()) == hipSuccess; };

    const dim3 tgrid((unsigned)(p / 32), (unsigned)(n / 32), (unsigned)pairs);
    if (init_state)
        hipLaunchKernelGGL(k_transpose_tiles, tgrid, dim3(256), 0, s, init_state, w.initT,
                           (int)n, (int)p);
    if (d_final)
        hipLaunchKernelGGL(k_transpose_tiles, tgrid, dim3(256), 0, s, d_final, w.dfT, (int)n,
                           (int)p);
    if (!ok()) return SSD_ERR_HIP;

    // 1. the adjoint, reversed: read-out yb_t = g_t^T B_t, final state g_0
    bf16 *y1 = reinterpret_cast<bf16 *>(ws + P.y1), *y2 = reinterpret_cast<bf16 *>(ws + P.y2);
    bf16 *y3 = reinterpret_cast<bf16 *>(ws + P.y3);
    float *du = reinterpret_cast<float *>(ws + P.du), *dw = reinterpret_cast<float *>(ws + P.dw);
    // the two adjoint scans share their chunks (scan 3 reads scan 1's states)
    const int m = state_interval(P.s1, false, bf16_item_heads(p, h, g));
    ScanArgs a1{dy, dt, C, B, A, nullptr, dt_bias, sp, dt_min, dt_max, d_final, y1,
                d_init ? w.fin1 : nullptr, scan_ws, seq_idx, nullptr};
    a1.adj = 1;
    a1.rev = 1;
    a1.dshift = 1;
    a1.interval = m;
    if ((e = scan_bf16(P.s1, a1, s)) != hipSuccess) return SSD_ERR_HIP;
    // 3. the adjoint transposed, reversed (x slot: the head's group row of
    //    C): its boundary states are scan 1's, read transposed; read-out
    //    g_t x_t and its dot with B_t (yb_t . x_t)
    ScanArgs a3{C, dt, dy, x, A, nullptr, dt_bias, sp, dt_min, dt_max, d_final, y3, nullptr,
                scan_ws, seq_idx, nullptr};
    a3.xrow = g * n;
    a3.xdiv = (int)(h / g);
    a3.adj = 1;
    a3.rev = 1;
    a3.dshift = 1;
    a3.dotv = B;
    a3.dotrow = g * n;
    a3.dotdiv = (int)(h / g);
    a3.dotout = dw;
    a3.interval = m;
    if ((P.s1.l + m * P.s1.Q - 1) / (m * P.s1.Q) > 1) {
        a3.hb_in = scan_ws + P.s1.off_hb;
        a3.hs_in = reinterpret_cast<const float *>(scan_ws + P.s1.off_hs);
        a3.hbt = 1;
    } else {
        // one chunk: scan 1 stored no states; scan 3 starts from d_final^T
        a3.init = d_final ? w.dfT : nullptr;
    }
    if ((e = scan_bf16(P.s2, a3, s)) != hipSuccess) return SSD_ERR_HIP;
    // 2. the forward transposed (x slot: the head's group row of B): read-out
    //    h_t dy_t, its dot with C_t (u), final state h_l^T
    ScanArgs a2{B, dt, x, dy, A, nullptr, dt_bias, sp, dt_min, dt_max,
                init_state ? w.initT : nullptr, y2, d_final ? w.finT : nullptr, scan_ws,
                seq_idx, nullptr};
    a2.xrow = g * n;
    a2.xdiv = (int)(h / g);
    a2.dotv = C;
    a2.dotrow = g * n;
    a2.dotdiv = (int)(h / g);
    a2.dotout = du;
    if ((e = scan_bf16(P.s2, a2, s)) != hipSuccess) return SSD_ERR_HIP;

    hipLaunchKernelGGL(k_bwd_tokg, dim3((unsigned)bl), dim3(256), 0, s, x, dt, dy, D, dt_bias,
                       sp, dt_min, dt_max, y1, y2, y3, du, dw, P.nparts, w.sc, dx, dB, dC, l,
                       (int)h, (int)g, (int)p, (int)n);
    hipLaunchKernelGGL((k_bwd_cum<bf16>), dim3((unsigned)pairs), dim3(kCumThreads), 0, s, dt, A,
                       dt_bias, sp, dt_min, dt_max, seq_idx, init_state ? 1 : 0, w, ddt, l,
                       (int)h, d_final ? w.dfT : nullptr, d_final ? w.finT : nullptr, np);
    hipLaunchKernelGGL(k_bwd_sum, dim3((unsigned)((h + 63) / 64)), dim3(64), 0, s, w.part, dA,
                       d_dt_bias, dD, b, (int)h);
    if (d_init)
        hipLaunchKernelGGL(k_bwd_init, dim3(eblk), dim3(256), 0, s, w.fin1, w.sc, A, d_init,
                           pairs, (int)h, l, np);
    return ok() ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

}  // namespace ssd

using namespace ssd;

extern "C" {

size_t ssd_chunk_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads,
                                          int64_t head_dim, int64_t state_dim, int64_t groups,
                                          int64_t chunk, int32_t io_dtype) {
    if (io_dtype == SSD_BF16) {
        BwdPlan16 P;
        if (!make_bwd_plan16(P, batch, seqlen, heads, head_dim, state_dim, groups, chunk))
            return 0;
        return P.total;
    }
    if (io_dtype != SSD_F32) return 0;
    BwdPlan P;
    if (!make_bwd_plan(P, batch, seqlen, heads, head_dim, state_dim, groups, chunk)) return 0;
    return P.total;
}

int32_t ssd_chunk_scan_bwd(const void *x, const void *dt, const float *A, const void *B,
                           const void *C, const float *D, const float *dt_bias,
                           int32_t dt_softplus, float dt_min, float dt_max,
                           const float *init_state, const int32_t *seq_idx, const void *dy,
                           const float *d_final, void *dx, void *ddt, float *dA, void *dB,
                           void *dC, float *dD, float *d_dt_bias, float *d_init, int64_t batch,
                           int64_t seqlen, int64_t heads, int64_t head_dim, int64_t state_dim,
                           int64_t groups, int64_t chunk, int32_t io_dtype, void *workspace,
                           size_t workspace_bytes, void *hip_stream) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (batch <= 0 || seqlen <= 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0 ||
        groups <= 0 || chunk <= 0 || heads % groups != 0)
        return SSD_ERR_SHAPE;
    // the transposed scans take head_dim as their state size
    const bool dims = (head_dim == 32 || head_dim == 64 || head_dim == 128) &&
                      (state_dim == 32 || state_dim == 64 || state_dim == 128);
    if (!dims) return SSD_ERR_UNSUPPORTED;
    const int64_t lim32 = (int64_t)1 << 31;
    if (batch * seqlen > lim32 / 2 || 64 * heads * 128 * 4 >= lim32 ||
        batch * seqlen * heads * 128 >= ((int64_t)1 << 40))
        return SSD_ERR_UNSUPPORTED;
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC)
        return SSD_ERR_NULL;
    const uintptr_t es = io_dtype == SSD_BF16 ? 2 : 4;
    if (!al16(x) || !al16(B) || !al16(C) || !al16(dy) || !al16(dx) || !al16(dB) || !al16(dC) ||
        !al16(init_state) || !al16(d_final) || !al16(d_init) || !al16(workspace) ||
        ((uintptr_t)dt % es) || ((uintptr_t)ddt % es) || ((uintptr_t)seq_idx & 3) ||
        ((uintptr_t)A & 3) || ((uintptr_t)D & 3) || ((uintptr_t)dt_bias & 3) ||
        ((uintptr_t)dA & 3) || ((uintptr_t)dD & 3) || ((uintptr_t)d_dt_bias & 3))
        return SSD_ERR_ALIGN;
    if (io_dtype == SSD_BF16)
        return bwd_bf16(static_cast<const bf16 *>(x), static_cast<const bf16 *>(dt), A,
                        static_cast<const bf16 *>(B), static_cast<const bf16 *>(C), D, dt_bias,
                        dt_softplus, dt_min, dt_max, init_state, seq_idx,
                        static_cast<const bf16 *>(dy), d_final, static_cast<bf16 *>(dx),
                        static_cast<bf16 *>(ddt), dA, static_cast<bf16 *>(dB),
                        static_cast<bf16 *>(dC), dD, d_dt_bias, d_init, batch, seqlen, heads,
                        head_dim, state_dim, groups, chunk, workspace, workspace_bytes,
                        static_cast<hipStream_t>(hip_stream));
    BwdPlan P;
    if (!make_bwd_plan(P, batch, seqlen, heads, head_dim, state_dim, groups, chunk))
        return SSD_ERR_SHAPE;
    if (P.s1.lp * 4 >= lim32 || P.s2.lp * 4 >= lim32) return SSD_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < P.total) return SSD_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    char *ws = static_cast<char *>(workspace);
    BwdBufs w;
    w.dyR = reinterpret_cast<float *>(ws + P.dyR);
    w.xR = reinterpret_cast<float *>(ws + P.xR);
    w.xF = reinterpret_cast<float *>(ws + P.xF);
    w.dyF = reinterpret_cast<float *>(ws + P.dyF);
    w.CR = reinterpret_cast<float *>(ws + P.CR);
    w.BR = reinterpret_cast<float *>(ws + P.BR);
    w.Bh = reinterpret_cast<float *>(ws + P.Bh);
    w.CRh = reinterpret_cast<float *>(ws + P.CRh);
    w.dtF = reinterpret_cast<float *>(ws + P.dtF);
    w.lw = reinterpret_cast<float *>(ws + P.lw);
    w.la = reinterpret_cast<float *>(ws + P.la);
    w.seqR = reinterpret_cast<int32_t *>(ws + P.seqR);
    w.y1 = reinterpret_cast<float *>(ws + P.y1);
    w.y2 = reinterpret_cast<float *>(ws + P.y2);
    w.y3 = reinterpret_cast<float *>(ws + P.y3);
    w.sc = reinterpret_cast<float *>(ws + P.sc);
    w.part = reinterpret_cast<double *>(ws + P.part);
    w.term = d_final ? reinterpret_cast<double *>(ws + P.term) : nullptr;
    w.fin1 = reinterpret_cast<float *>(ws + P.fin1);
    w.finT = reinterpret_cast<float *>(ws + P.finT);
    w.initT = reinterpret_cast<float *>(ws + P.initT);
    w.dfT = reinterpret_cast<float *>(ws + P.dfT);
    char *scan_ws = ws + P.ws;

    const int64_t b = batch, l = seqlen, h = heads, p = head_dim, n = state_dim, g = groups;
    const int64_t bl = b * l, pairs = b * h, np = n * p;
    const unsigned eblk = (unsigned)((pairs * np + 255) / 256);
    const float inf = INFINITY;
    hipError_t e = hipSuccess;
    auto ok = [&]() { return (e = hipGetLastError()) == hipSuccess; };

    if (io_dtype == SSD_BF16)
        hipLaunchKernelGGL((k_bwd_prep<bf16>), dim3((unsigned)bl), dim3(256), 0, s,
                           static_cast<const bf16 *>(x), static_cast<const bf16 *>(dt), A,
                           static_cast<const bf16 *>(B), static_cast<const bf16 *>(C),
                           static_cast<const bf16 *>(dy), dt_bias, dt_softplus ? 1 : 0, dt_min,
                           dt_max, seq_idx, w, l, (int)h, (int)g, (int)p, (int)n);
    else
        hipLaunchKernelGGL((k_bwd_prep<float>), dim3((unsigned)bl), dim3(256), 0, s,
                           static_cast<const float *>(x), static_cast<const float *>(dt), A,
                           static_cast<const float *>(B), static_cast<const float *>(C),
                           static_cast<const float *>(dy), dt_bias, dt_softplus ? 1 : 0, dt_min,
                           dt_max, seq_idx, w, l, (int)h, (int)g, (int)p, (int)n);
    if (init_state)
        hipLaunchKernelGGL(k_transpose_np, dim3(eblk), dim3(256), 0, s, init_state, w.initT,
                           pairs, (int)n, (int)p);
    if (d_final)
        hipLaunchKernelGGL(k_transpose_np, dim3(eblk), dim3(256), 0, s, d_final, w.dfT, pairs,
                           (int)n, (int)p);
    if (!ok()) return SSD_ERR_HIP;

    // 1. the adjoint, reversed: read-out yb_t = g_t^T B_t, final state g_0
    ScanArgs a1{w.dyR, w.dtF, w.CR, w.BR, A, nullptr, nullptr, 0, 0.f, inf,
                d_final, w.y1, w.fin1, scan_ws, seq_idx ? w.seqR : nullptr, nullptr};
    a1.lw = w.lw;
    a1.la = w.la;
    if ((e = scan_f32(P.s1, a1, s)) != hipSuccess) return SSD_ERR_HIP;
    // 2. the forward transposed: read-out h_t dy_t, final state h_l^T
    ScanArgs a2{w.Bh, w.dtF, w.xF, w.dyF, A, nullptr, dt_bias, dt_softplus ? 1 : 0, dt_min,
                dt_max, init_state ? w.initT : nullptr, w.y2, d_final ? w.finT : nullptr,
                scan_ws, seq_idx, nullptr};
    if ((e = scan_f32(P.s2, a2, s)) != hipSuccess) return SSD_ERR_HIP;
    // 3. the adjoint transposed, reversed: read-out g_t x_t
    ScanArgs a3{w.CRh, w.dtF, w.dyR, w.xR, A, nullptr, nullptr, 0, 0.f, inf,
                d_final ? w.dfT : nullptr, w.y3, nullptr, scan_ws,
                seq_idx ? w.seqR : nullptr, nullptr};
    a3.lw = w.lw;
    a3.la = w.la;
    if ((e = scan_f32(P.s2, a3, s)) != hipSuccess) return SSD_ERR_HIP;

    const unsigned tblk = (unsigned)((bl * h + 15) / 16);
    if (io_dtype == SSD_BF16)
        hipLaunchKernelGGL((k_bwd_tok<bf16>), dim3(tblk), dim3(256), 0, s,
                           static_cast<const bf16 *>(x), static_cast<const bf16 *>(dt),
                           static_cast<const bf16 *>(C), static_cast<const bf16 *>(dy), D,
                           dt_bias, dt_softplus ? 1 : 0, dt_min, dt_max, w,
                           static_cast<bf16 *>(dx), bl, l, (int)h, (int)g, (int)p, (int)n);
    else
        hipLaunchKernelGGL((k_bwd_tok<float>), dim3(tblk), dim3(256), 0, s,
                           static_cast<const float *>(x), static_cast<const float *>(dt),
                           static_cast<const float *>(C), static_cast<const float *>(dy), D,
                           dt_bias, dt_softplus ? 1 : 0, dt_min, dt_max, w,
                           static_cast<float *>(dx), bl, l, (int)h, (int)g, (int)p, (int)n);
    if (d_final)
        hipLaunchKernelGGL(k_bwd_term, dim3((unsigned)pairs), dim3(256), 0, s, d_final, w.finT,
                           w.term, (int)n, (int)p);
    if (io_dtype == SSD_BF16)
        hipLaunchKernelGGL((k_bwd_cum<bf16>), dim3((unsigned)pairs), dim3(kCumThreads), 0, s,
                           static_cast<const bf16 *>(dt), A, dt_bias, dt_softplus ? 1 : 0,
                           dt_min, dt_max, seq_idx, init_state ? 1 : 0, w,
                           static_cast<bf16 *>(ddt), l, (int)h);
    else
        hipLaunchKernelGGL((k_bwd_cum<float>), dim3((unsigned)pairs), dim3(kCumThreads), 0, s,
                           static_cast<const float *>(dt), A, dt_bias, dt_softplus ? 1 : 0,
                           dt_min, dt_max, seq_idx, init_state ? 1 : 0, w,
                           static_cast<float *>(ddt), l, (int)h);
    if (io_dtype == SSD_BF16)
        hipLaunchKernelGGL((k_bwd_group<bf16>), dim3((unsigned)bl), dim3(256), 0, s, w,
                           static_cast<bf16 *>(dB), static_cast<bf16 *>(dC), l, (int)h, (int)g,
                           (int)n);
    else
        hipLaunchKernelGGL((k_bwd_group<float>), dim3((unsigned)bl), dim3(256), 0, s, w,
                           static_cast<float *>(dB), static_cast<float *>(dC), l, (int)h, (int)g,
                           (int)n);
    hipLaunchKernelGGL(k_bwd_sum, dim3((unsigned)((h + 63) / 64)), dim3(64), 0, s, w.part, dA,
                       d_dt_bias, dD, b, (int)h);
    if (d_init)
        hipLaunchKernelGGL(k_bwd_init, dim3(eblk), dim3(256), 0, s, w.fin1, w.sc, A, d_init,
                           pairs, (int)h, l, np);
    return ok() ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
