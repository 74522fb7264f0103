// The chunked SSD scan on gfx950: kernels and their launch sequence.
//
// The recurrence (nnterp guide, "Mamba-2" page, opening section)
//     h_t = exp(a_t) h_{t-1} + d_t B_t x_t^T,   y_t = C_t^T h_t + D x_t,
// a_t = A d_t, is evaluated in the two-stage chunked form of the kongchang
// "Mamba2" page (chunk-scan entry): inside a chunk everything is matrix
// products on the matrix cores; across chunks one serial pass carries the
// state, and the state entering every chunk is stored as one boundary-state
// tensor (nnterp, "The state after every token").
//
// Rows are handled in blocks of kT = 32 rows that never straddle a chunk
// boundary.  With lcs_i the cumulative log2 decay inside a block (inclusive)
// and H the state entering the block:
//   y_i = sum_{j<=i} (C_i . B_j) 2^(lcs_i - lcs_j) d_j x_j
//         + 2^lcs_i C_i^T H + D x_i                          (intra + read)
//   H'  = 2^lcs_last H + sum_j B_j (2^(lcs_last - lcs_j) d_j x_j)^T   (write)
// Every exponent is <= 0 when A <= 0; the j > i half is removed by a select
// before any exponential is taken, so no inf * 0 can arise.
//
// Launch sequence on one stream:
//   1. k_dt_cumsum   d, and lcs per block                      (row a1)
//   2. k_state_pass  chunk states on the matrix cores, serial over chunks
//                    inside a segment; writes the boundary states (rows a2, a3)
//   3. k_seg_combine only when the sequence is cut into several segments:
//                    carries the state across segment ends     (row a3)
//   4. k_chunk_out   per (batch, chunk, head): intra-chunk masked product,
//                    read of the boundary state, skip term     (rows a4, a5)
#pragma once

#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

constexpr int kT = 32;  // rows per block

// ----------------------------------------------------------------------------
// 1. Time step and per-block cumulative log2 decay.
//    grid (chunks, batch, ceil(heads / 4)); one wave per head.
//    lcs[b, h, c*Qp + r] = log2(e) * sum_{k = block start .. r} A d_k
//    dtp[b, h, c*Qp + r] = d_r   (0 on padded rows)
template <typename IO>
__global__ __launch_bounds__(256) void k_dt_cumsum(
    const IO *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ dt_bias,
    int softplus, float dt_min, float dt_max, int64_t l, int h, int64_t Q, int64_t nc,
    int64_t Qp, float *__restrict__ lcs, float *__restrict__ dtp) {
    constexpr int T = kT;
    const int64_t c = blockIdx.x, b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int hh = blockIdx.z * kWaves + wave;
    if (hh >= h) return;
    const float a2 = A[hh] * kLog2e;
    const float bias = dt_bias ? dt_bias[hh] : 0.f;
    const int64_t base = ((b * h + hh) * nc + c) * Qp;
    for (int64_t r0 = 0; r0 < Qp; r0 += 64) {
        const int64_t rp = r0 + lane;
        const int64_t t = c * Q + rp;
        float d = 0.f;
        if (rp < Q && t < l)
            d = time_step(to_f32(dt[(b * l + t) * h + hh]), bias, softplus, dt_min, dt_max);
        float a = a2 * d;
#pragma unroll
        for (int off = 1; off < T; off <<= 1) {
            const float v = __shfl_up(a, off, T);
            if ((lane & (T - 1)) >= off) a += v;
        }
        if (rp < Qp) {
            lcs[base + rp] = a;
            dtp[base + rp] = d;
        }
    }
}

// ----------------------------------------------------------------------------
// Staging of the state pass: one slab = SLAB blocks of kT rows.  Pieces are
// 8 consecutive elements of one row of x (P / 8 per row) or of the
// workgroup's NW-column slice of B (NW / 8 per row).  The prefetch only
// issues loads (row index clamped to a readable row) and records which
// pieces are real rows; conversions and selects happen in the stage step,
// so nothing waits on a load before it is needed.
template <typename IO, int P, int NW, int SLAB> struct SpBuf {
    static constexpr int NPX = SLAB * kT * P / 8, NPB = SLAB * kT * NW / 8;
    static constexpr int KX = (NPX + kThreads - 1) / kThreads;
    static constexpr int KB = (NPB + kThreads - 1) / kThreads;
    Row8v<IO> xv[KX], bv[KB];
    float xl[KX], xd[KX], xe[KX];  // lcs, d of the x piece's row; lcs at its block end
    float lam[SLAB];               // log2 decay of each block of the slab
    uint32_t okx, okb;             // bit k: piece k is a real row
};

template <typename IO, int P, int NW, int SLAB>
__device__ __forceinline__ void sp_prefetch(SpBuf<IO, P, NW, SLAB> &f, int64_t s0, int64_t sb1,
                                            int64_t nsb, const IO *xb, const IO *Bb,
                                            const float *lcs_bh, const float *dtp_bh, int64_t l,
                                            int64_t Q, int64_t xstride, int64_t bstride, int tid) {
    typedef SpBuf<IO, P, NW, SLAB> F;
    constexpr int T = kT;
    const int nb = (int)((sb1 - s0) < SLAB ? (sb1 - s0) : SLAB);
    f.okx = 0;
    f.okb = 0;
#pragma unroll
    for (int k = 0; k < F::KX; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPX % kThreads == 0 || q < F::NPX) {
            const int j = q / (P / 8), cc = q % (P / 8), jb = j / T;
            const int64_t sb = s0 + (jb < nb ? jb : 0);
            const int64_t rp = (sb % nsb) * T + (j % T), t = (sb / nsb) * Q + rp;
            const bool ok = jb < nb && rp < Q && t < l;
            f.xv[k] = ld_row8(xb + (ok ? t : 0) * xstride + cc * 8);
            const int64_t R = sb * T + (j % T);
            f.xl[k] = lcs_bh[R];
            f.xd[k] = dtp_bh[R];
            f.xe[k] = lcs_bh[sb * T + T - 1];
            f.okx |= (uint32_t)ok << k;
        }
    }
#pragma unroll
    for (int k = 0; k < F::KB; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPB % kThreads == 0 || q < F::NPB) {
            const int j = q / (NW / 8), cc = q % (NW / 8), jb = j / T;
            const int64_t sb = s0 + (jb < nb ? jb : 0);
            const int64_t rp = (sb % nsb) * T + (j % T), t = (sb / nsb) * Q + rp;
            const bool ok = jb < nb && rp < Q && t < l;
            f.bv[k] = ld_row8(Bb + (ok ? t : 0) * bstride + cc * 8);
            f.okb |= (uint32_t)ok << k;
        }
    }
#pragma unroll
    for (int jb = 0; jb < SLAB; ++jb) f.lam[jb] = lcs_bh[(s0 + (jb < nb ? jb : 0)) * T + T - 1];
}

template <typename IO, int P, int NW, int SLAB>
__device__ __forceinline__ void sp_stage(const SpBuf<IO, P, NW, SLAB> &f,
                                         typename Op<IO>::type *Xw,
                                         typename Op<IO>::type *Bs, int tid) {
    typedef SpBuf<IO, P, NW, SLAB> F;
    constexpr int LDX = P + 16, LDB = NW + 16;
#pragma unroll
    for (int k = 0; k < F::KX; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPX % kThreads == 0 || q < F::NPX) {
            const bool ok = (f.okx >> k) & 1;
            const float w = ok ? exp2_fast(f.xe[k] - f.xl[k]) * f.xd[k] : 0.f;
            st_row8(Xw + (q / (P / 8)) * LDX + (q % (P / 8)) * 8, to_op_scaled(f.xv[k], w));
        }
    }
#pragma unroll
    for (int k = 0; k < F::KB; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPB % kThreads == 0 || q < F::NPB)
            st_row8(Bs + (q / (NW / 8)) * LDB + (q % (NW / 8)) * 8,
                    to_op(f.bv[k], (f.okb >> k) & 1));
    }
}

// ----------------------------------------------------------------------------
// 2. Chunk states and the serial pass over chunks.
//    One workgroup per (batch, segment, head, NW-row slice of the state).  The
//    slice H[n0:n0+NW, :] lives in MFMA accumulators for the whole segment.
//    Each iteration takes a slab of up to SLAB row blocks: B (raw) and the
//    decay-weighted x (w_j x_j, w_j = 2^(lcs_last - lcs_j) d_j) are copied row
//    by row into LDS while the next slab is already being fetched, then block
//    by block
//        H <- 2^lcs_last H + B^T (w x)      (contraction over the block rows)
//    with both operands read k-major through transposing LDS loads.  Before
//    the first block of every chunk the slice is written out as that chunk's
//    boundary state.  Segment 0 starts from init_state; later segments start
//    from zero and are corrected by k_seg_combine and in k_chunk_out.
template <typename IO, int P, int N>
__global__ __launch_bounds__(256) void k_state_pass(
    const IO *__restrict__ x, const IO *__restrict__ Bm, const float *__restrict__ lcs,
    const float *__restrict__ dtp, const float *__restrict__ init, float *__restrict__ Hb,
    float *__restrict__ Eseg, float *__restrict__ Dlog, float *__restrict__ Lseg,
    float *__restrict__ final_state, int64_t l, int h, int g, int64_t Q, int64_t nc,
    int64_t Qp, int64_t cps, int64_t nseg) {
    typedef typename Op<IO>::type OP;
    typedef Mfma<OP> M;
    constexpr int T = kT;
    constexpr int KS = T / M::K;            // MFMA steps per block
    constexpr int NW = 32;                  // state rows per workgroup
    constexpr int NSPLIT = N / NW;
    constexpr int SLAB = 4;                 // blocks per iteration
    constexpr int SR = SLAB * T;            // rows per slab
    constexpr int LDX = P + 16, LDB = NW + 16;
    constexpr int TILES = (NW / 16) * (P / 16);
    constexpr int TPW = (TILES + kWaves - 1) / kWaves;
    __shared__ __attribute__((aligned(16))) OP Xw[SR * LDX];  // w x  [row][p]
    __shared__ __attribute__((aligned(16))) OP Bs[SR * LDB];  // B    [row][n - n0]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int split = (int)(item % NSPLIT); item /= NSPLIT;
    const int hh = (int)(item % h); item /= h;
    const int64_t seg = item % nseg;
    const int64_t b = item / nseg;
    const int gi = hh / (h / g);
    const int n0 = split * NW;
    const int64_t nsb = Qp / T;
    const int64_t c0 = seg * cps;
    const int64_t c1 = (c0 + cps < nc) ? c0 + cps : nc;
    const int64_t sb0 = c0 * nsb, sb1 = c1 * nsb;
    const float *lcs_bh = lcs + (b * h + hh) * nc * Qp;
    const float *dtp_bh = dtp + (b * h + hh) * nc * Qp;
    const int64_t NP = (int64_t)N * P;

    f32x4 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = zero4();
    if (seg == 0 && init) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int ti = wave + kWaves * i;
            const int tr = ti / (P / 16), tc = ti % (P / 16);
            const float *src = init + (b * h + hh) * NP +
                               (int64_t)(n0 + tr * 16 + 4 * (lane >> 4)) * P + tc * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = ti < TILES ? src[r * P] : 0.f;
        }
    }
    float logdec = 0.f;

    SpBuf<IO, P, NW, SLAB> pf;
    const IO *xb = x + (b * l * h + hh) * P;         // row t at xb + t * h * P
    const IO *Bb = Bm + (b * l * g + gi) * N + n0;    // row t at Bb + t * g * N
    if (sb0 < sb1)
        sp_prefetch(pf, sb0, sb1, nsb, xb, Bb, lcs_bh, dtp_bh, l, Q, (int64_t)h * P,
                    (int64_t)g * N, tid);
    for (int64_t s0 = sb0; s0 < sb1; s0 += SLAB) {
        const int nb = (int)((sb1 - s0) < SLAB ? (sb1 - s0) : SLAB);
        float lam[SLAB];
#pragma unroll
        for (int jb = 0; jb < SLAB; ++jb) lam[jb] = pf.lam[jb];
        sp_stage(pf, Xw, Bs, tid);
        if (s0 + SLAB < sb1)
            sp_prefetch(pf, s0 + SLAB, sb1, nsb, xb, Bb, lcs_bh, dtp_bh, l, Q, (int64_t)h * P,
                        (int64_t)g * N, tid);
        lds_barrier();
        for (int jb = 0; jb < nb; ++jb) {
            const int64_t sb = s0 + jb;
            if (sb % nsb == 0) {  // first block of a chunk: emit the boundary state
                const int64_t c = sb / nsb;
                float *dst = Hb + ((b * nc + c) * h + hh) * NP;
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int ti = wave + kWaves * i;
                    if (ti < TILES) {
                        const int tr = ti / (P / 16), tc = ti % (P / 16);
                        float *d0 = dst + (int64_t)(n0 + tr * 16 + 4 * (lane >> 4)) * P +
                                    tc * 16 + (lane & 15);
#pragma unroll
                        for (int r = 0; r < 4; ++r) d0[r * P] = acc[i][r];
                    }
                }
                if (nseg > 1 && split == 0 && tid == 0) Dlog[(b * h + hh) * nc + c] = logdec;
            }
            const float decay = exp2_fast(lam[jb]);
            logdec += lam[jb];
#pragma unroll
            for (int i = 0; i < TPW; ++i) acc[i] *= decay;
#pragma unroll
            for (int q = 0; q < KS; ++q) {
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int ti = wave + kWaves * i;
                    if (ti < TILES) {
                        const int tr = ti / (P / 16), tc = ti % (P / 16);
                        acc[i] = M::mma(frag_kmajor(Bs, LDB, jb * T, q, tr * 16, lane),
                                        frag_kmajor(Xw, LDX, jb * T, q, tc * 16, lane), acc[i]);
                    }
                }
            }
        }
        lds_barrier();
    }

    float *out = nullptr;
    if (nseg == 1)
        out = final_state ? final_state + (b * h + hh) * NP : nullptr;
    else
        out = Eseg + ((b * nseg + seg) * h + hh) * NP;
    if (out) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int ti = wave + kWaves * i;
            if (ti < TILES) {
                const int tr = ti / (P / 16), tc = ti % (P / 16);
                float *d0 = out + (int64_t)(n0 + tr * 16 + 4 * (lane >> 4)) * P + tc * 16 +
                            (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) d0[r * P] = acc[i][r];
            }
        }
    }
    if (nseg > 1 && split == 0 && tid == 0) Lseg[(b * h + hh) * nseg + seg] = logdec;
}

// ----------------------------------------------------------------------------
// 3. Segment combine: the state entering segment k (k >= 1) is
//        Hin_k = 2^L_{k-1} Hin_{k-1} + E_{k-1},   Hin_1 = E_0,
//    with E_k the state segment k reaches from zero (segment 0 from the
//    initial state) and L_k its total log2 decay.  Hin_k overwrites slot
//    k - 1 of Eseg; the state after the last segment is the final state.
//    One thread per 4 consecutive state elements of one (batch, head).
static __global__ __launch_bounds__(256) void k_seg_combine(float *__restrict__ Eseg,
                                                     const float *__restrict__ Lseg,
                                                     float *__restrict__ final_state,
                                                     int64_t bh, int h, int64_t nseg,
                                                     int64_t np4) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= bh * np4) return;
    const int64_t pair = idx / np4, e4 = idx % np4;
    const int64_t b = pair / h, hh = pair % h;
    f32x4 *E = reinterpret_cast<f32x4 *>(Eseg) + (b * nseg * h + hh) * np4 + e4;
    const int64_t stride = (int64_t)h * np4;  // from one segment slot to the next
    f32x4 H = E[0];
    for (int64_t k = 1; k < nseg; ++k) {
        const f32x4 Ek = E[k * stride];
        E[(k - 1) * stride] = H;
        H = exp2_fast(Lseg[pair * nseg + k]) * H + Ek;
    }
    if (final_state) reinterpret_cast<f32x4 *>(final_state)[pair * np4 + e4] = H;
}

// ----------------------------------------------------------------------------
// Staging of the chunk output: one block of kT rows.  Pieces are 8
// consecutive elements of one row of C and of B (same row and columns, N / 8
// per row) or of x (P / 8 per row).  As in the state pass, the prefetch only
// issues loads and records which pieces are real rows.
template <typename IO, int P, int N> struct CoBuf {
    static constexpr int NPC = kT * N / 8, NPX = kT * P / 8;
    static constexpr int KC = (NPC + kThreads - 1) / kThreads;
    static constexpr int KX = (NPX + kThreads - 1) / kThreads;
    Row8v<IO> cv[KC], bv[KC], xv[KX];
    float xl[KX], xd[KX];  // lcs and d of the x piece's row
    float last, ls, ds;    // lcs at the block end; lcs and d of row tid (tid < kT)
    uint32_t okc, okx;
};

template <typename IO, int P, int N>
__device__ __forceinline__ void co_prefetch(CoBuf<IO, P, N> &f, int s, const IO *xb,
                                            const IO *Bb, const IO *Cb, const float *lcs_c,
                                            const float *dtp_c, int64_t t0, int64_t l, int64_t Q,
                                            int64_t xstride, int64_t bstride, int tid) {
    typedef CoBuf<IO, P, N> F;
    constexpr int T = kT;
    const int64_t rpb = (int64_t)s * T;
    f.okc = 0;
    f.okx = 0;
#pragma unroll
    for (int k = 0; k < F::KC; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPC % kThreads == 0 || q < F::NPC) {
            const int j = q / (N / 8), cc = q % (N / 8);
            const int64_t rp = rpb + j, t = t0 + rp;
            const bool ok = rp < Q && t < l;
            const int64_t off = (ok ? t : 0) * bstride + cc * 8;
            f.cv[k] = ld_row8(Cb + off);
            f.bv[k] = ld_row8(Bb + off);
            f.okc |= (uint32_t)ok << k;
        }
    }
#pragma unroll
    for (int k = 0; k < F::KX; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPX % kThreads == 0 || q < F::NPX) {
            const int j = q / (P / 8), cc = q % (P / 8);
            const int64_t rp = rpb + j, t = t0 + rp;
            const bool ok = rp < Q && t < l;
            f.xv[k] = ld_row8(xb + (ok ? t : 0) * xstride + cc * 8);
            f.xl[k] = lcs_c[rp];
            f.xd[k] = dtp_c[rp];
            f.okx |= (uint32_t)ok << k;
        }
    }
    f.last = lcs_c[rpb + T - 1];
    const int64_t rt = rpb + (tid < T ? tid : 0);
    f.ls = lcs_c[rt];
    f.ds = dtp_c[rt];
}

template <typename IO, int P, int N>
__device__ __forceinline__ void co_stage(const CoBuf<IO, P, N> &f, typename Op<IO>::type *Cs,
                                         typename Op<IO>::type *Bs, typename Op<IO>::type *Xs,
                                         typename Op<IO>::type *Xw, float *lcs_s, float *d_s,
                                         int tid) {
    typedef CoBuf<IO, P, N> F;
    typedef typename Op<IO>::type OP;
    constexpr int LDN = N + Mfma<OP>::PAD, LDX = P + 16;
#pragma unroll
    for (int k = 0; k < F::KC; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPC % kThreads == 0 || q < F::NPC) {
            const int o = (q / (N / 8)) * LDN + (q % (N / 8)) * 8;
            const bool ok = (f.okc >> k) & 1;
            st_row8(Cs + o, to_op(f.cv[k], ok));
            st_row8(Bs + o, to_op(f.bv[k], ok));
        }
    }
#pragma unroll
    for (int k = 0; k < F::KX; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPX % kThreads == 0 || q < F::NPX) {
            const int o = (q / (P / 8)) * LDX + (q % (P / 8)) * 8;
            const bool ok = (f.okx >> k) & 1;
            st_row8(Xs + o, to_op(f.xv[k], ok));
            const float w = ok ? exp2_fast(f.last - f.xl[k]) * f.xd[k] : 0.f;
            st_row8(Xw + o, to_op_scaled(f.xv[k], w));
        }
    }
    if (tid < kT) {
        lcs_s[tid] = f.ls;
        d_s[tid] = f.ds;
    }
}

// ----------------------------------------------------------------------------
// 4. Chunk output.  One workgroup per (batch, chunk, head); the blocks of the
//    chunk are taken in order with the running state H in MFMA accumulators
//    (fp32) and, as the operand copy H^T, in LDS.  Per block, with C, B, x and
//    the decay-weighted x staged row by row while the next block is already
//    being fetched:
//      G^T = B C^T on the causal tiles of the wave's row strip, and
//      P_ij = G_ij 2^(lcs_i - lcs_j) d_j (j <= i), kept in registers;
//      Y = 2^lcs_i (C H) + P x + D x, written to y;
//      H <- 2^lcs_last H + B^T (w x)  (except after the last block).
//    Two workgroup barriers per block.
template <typename IO, int P, int N>
__global__ __launch_bounds__(256) void k_chunk_out(
    const IO *__restrict__ x, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ lcs, const float *__restrict__ dtp,
    const float *__restrict__ Hb, const float *__restrict__ Hin, const float *__restrict__ Dlog,
    IO *__restrict__ y, int64_t l, int h, int g, int64_t Q, int64_t nc, int64_t Qp,
    int64_t cps, int64_t nseg) {
    typedef typename Op<IO>::type OP;
    typedef Mfma<OP> M;
    constexpr int T = kT;
    constexpr int KS = T / M::K;          // MFMA steps over the block rows
    constexpr int NS = N / M::K;          // MFMA steps over the state index
    constexpr int LDN = N + M::PAD;       // [row][n]: C, B (row-major and k-major), H^T
    constexpr int LDX = P + 16;           // k-major [row][p]: x, w x
    constexpr int CT = P / 16;            // column tiles of y and H
    constexpr int HTILES = (N / 16) * CT;
    constexpr int HPW = (HTILES + kWaves - 1) / kWaves;
    constexpr int YPW = CT >= 2 ? CT / 2 : 1;  // y tiles per wave (one row strip)
    __shared__ __attribute__((aligned(16))) OP Cs[T * LDN];   // C    [row][n]
    __shared__ __attribute__((aligned(16))) OP Bs[T * LDN];   // B    [row][n]
    __shared__ __attribute__((aligned(16))) OP Xs[T * LDX];   // x    [row][p]
    __shared__ __attribute__((aligned(16))) OP Xw[T * LDX];   // w x  [row][p]
    __shared__ __attribute__((aligned(16))) OP HT[P * LDN];   // H^T  [p][n]
    __shared__ float lcs_s[T];
    __shared__ float d_s[T];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, li = lane & 15;
    int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int hh = (int)(item % h); item /= h;
    const int64_t c = item % nc;
    const int64_t b = item / nc;
    const int gi = hh / (h / g);
    const int64_t seg = c / cps;
    const int64_t NP = (int64_t)N * P;
    const float *lcs_c = lcs + ((b * h + hh) * nc + c) * Qp;
    const float *dtp_c = dtp + ((b * h + hh) * nc + c) * Qp;
    const float Dh = D ? D[hh] : 0.f;
    const int64_t rows = (Q < l - c * Q) ? Q : (l - c * Q);  // valid rows of this chunk
    const int nblk = (int)((rows + T - 1) / T);
    // the wave's row strip and y tiles
    const bool yact = CT >= 2 || wave < 2;
    const int it = CT >= 2 ? (wave >> 1) : wave;
    const int pt0 = CT >= 2 ? (wave & 1) * (CT / 2) : 0;

    CoBuf<IO, P, N> pf;
    const IO *xb = x + (b * l * h + hh) * P;        // row t at xb + t * h * P
    const IO *Bb = Bm + (b * l * g + gi) * N;        // row t at Bb + t * g * N
    const IO *Cb = Cm + (b * l * g + gi) * N;
    if (nblk > 0)
        co_prefetch(pf, 0, xb, Bb, Cb, lcs_c, dtp_c, c * Q, l, Q, (int64_t)h * P, (int64_t)g * N,
                    tid);

    // ---- state entering the chunk (all loads issued before any is used)
    f32x4 accH[HPW];
    {
        const float *hb = Hb + ((b * nc + c) * h + hh) * NP;
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int ti = wave + kWaves * i;
            const int tr = ti / CT, tc = ti % CT;
            const int64_t off = (int64_t)(tr * 16 + 4 * lg) * P + tc * 16 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) accH[i][r] = ti < HTILES ? hb[off + r * P] : 0.f;
        }
        if (seg > 0) {
            const float *hin = Hin + ((b * nseg + seg - 1) * h + hh) * NP;
            f32x4 iv[HPW];
#pragma unroll
            for (int i = 0; i < HPW; ++i) {
                const int ti = wave + kWaves * i;
                const int tr = ti / CT, tc = ti % CT;
                const int64_t off = (int64_t)(tr * 16 + 4 * lg) * P + tc * 16 + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) iv[i][r] = ti < HTILES ? hin[off + r * P] : 0.f;
            }
            const float corr = exp2_fast(Dlog[(b * h + hh) * nc + c]);
#pragma unroll
            for (int i = 0; i < HPW; ++i) accH[i] += corr * iv[i];
        }
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int ti = wave + kWaves * i;
            if (ti < HTILES) {
                const int tr = ti / CT, tc = ti % CT;
                lds_store4(HT + (tc * 16 + li) * LDN + tr * 16 + 4 * lg, accH[i]);
            }
        }
    }

    for (int s = 0; s < nblk; ++s) {
        const int64_t rpb = (int64_t)s * T;
        co_stage(pf, Cs, Bs, Xs, Xw, lcs_s, d_s, tid);
        if (s + 1 < nblk)
            co_prefetch(pf, s + 1, xb, Bb, Cb, lcs_c, dtp_c, c * Q, l, Q, (int64_t)h * P,
                        (int64_t)g * N, tid);
        lds_barrier();

        if (yact) {
            // ---- masked, decayed scores of the wave's row strip (registers)
            const int i = it * 16 + li;
            const float li_cs = lcs_s[i];
            f32x4 pv[2];
            pv[0] = zero4();
            pv[1] = zero4();
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                if (jt <= it) {
                    f32x4 gacc = zero4();
#pragma unroll
                    for (int ks = 0; ks < NS; ++ks)
                        gacc = M::mma(lds_frag(Bs, LDN, jt * 16, ks * M::K, lane),
                                      lds_frag(Cs, LDN, it * 16, ks * M::K, lane), gacc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = jt * 16 + 4 * lg + r;
                        pv[jt][r] = (j <= i) ? gacc[r] * exp2_fast(li_cs - lcs_s[j]) * d_s[j] : 0.f;
                    }
                }
            }
            // ---- y tiles of the strip
            const int i0 = it * 16 + 4 * lg;
            f32x4 rowscale;
#pragma unroll
            for (int r = 0; r < 4; ++r) rowscale[r] = exp2_fast(lcs_s[i0 + r]);
#pragma unroll
            for (int u = 0; u < YPW; ++u) {
                const int pt = pt0 + u;
                f32x4 ya = zero4();
#pragma unroll
                for (int ks = 0; ks < NS; ++ks)
                    ya = M::mma(lds_frag(Cs, LDN, it * 16, ks * M::K, lane),
                                lds_frag(HT, LDN, pt * 16, ks * M::K, lane), ya);
                ya *= rowscale;
#pragma unroll
                for (int q = 0; q < KS; ++q)
                    ya = M::mma(frag_from_acc<OP>(pv[0], pv[1], q),
                                frag_kmajor(Xs, LDX, 0, q, pt * 16, lane), ya);
                const f32x4 xv = lds_col4(Xs, LDX, it * 16, pt * 16, lane);  // rows i0 + r
                const int p = pt * 16 + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t rp = rpb + i0 + r, t = c * Q + rp;
                    if (rp < Q && t < l)
                        y[((b * l + t) * h + hh) * P + p] = from_f32<IO>(ya[r] + Dh * xv[r]);
                }
            }
        }

        // ---- carry the state to the next block of the chunk
        if (s + 1 < nblk) {
            const float decay = exp2_fast(lcs_s[T - 1]);
#pragma unroll
            for (int i = 0; i < HPW; ++i) accH[i] *= decay;
#pragma unroll
            for (int q = 0; q < KS; ++q) {
#pragma unroll
                for (int i = 0; i < HPW; ++i) {
                    const int ti = wave + kWaves * i;
                    if (ti < HTILES) {
                        const int tr = ti / CT, tc = ti % CT;
                        accH[i] = M::mma(frag_kmajor(Bs, LDN, 0, q, tr * 16, lane),
                                         frag_kmajor(Xw, LDX, 0, q, tc * 16, lane), accH[i]);
                    }
                }
            }
        }
        lds_barrier();  // every read of this block's operands is done
        if (s + 1 < nblk) {
#pragma unroll
            for (int i = 0; i < HPW; ++i) {
                const int ti = wave + kWaves * i;
                if (ti < HTILES) {
                    const int tr = ti / CT, tc = ti % CT;
                    lds_store4(HT + (tc * 16 + li) * LDN + tr * 16 + 4 * lg, accH[i]);
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------
template <typename IO, int P, int N>
hipError_t launch_scan(const ScanPlan &pl, const ScanArgs &a, hipStream_t s) {
    float *lcs = reinterpret_cast<float *>(a.ws + pl.off_lcs);
    float *dtp = reinterpret_cast<float *>(a.ws + pl.off_dtp);
    float *Hb = reinterpret_cast<float *>(a.ws + pl.off_hb);
    float *Eseg = reinterpret_cast<float *>(a.ws + pl.off_seg);
    float *Dlog = reinterpret_cast<float *>(a.ws + pl.off_dlog);
    float *Lseg = reinterpret_cast<float *>(a.ws + pl.off_lseg);
    const IO *x = static_cast<const IO *>(a.x);
    const IO *dt = static_cast<const IO *>(a.dt);
    const IO *Bm = static_cast<const IO *>(a.B);
    const IO *Cm = static_cast<const IO *>(a.C);
    IO *y = static_cast<IO *>(a.y);
    const int h = (int)pl.h, g = (int)pl.g;

    trace_begin(0, s);
    hipLaunchKernelGGL(k_dt_cumsum<IO>, dim3((unsigned)pl.nc, (unsigned)pl.b, (unsigned)((h + 3) / 4)),
                       dim3(256), 0, s, dt, a.A, a.dt_bias, a.softplus, a.dt_min, a.dt_max, pl.l, h,
                       pl.Q, pl.nc, pl.Qp, lcs, dtp);
    trace_end(0, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int64_t nblk2 = pl.b * pl.nseg * pl.h * (N / 32);
    trace_begin(1, s);
    hipLaunchKernelGGL((k_state_pass<IO, P, N>), dim3((unsigned)nblk2), dim3(256), 0, s, x, Bm, lcs,
                       dtp, a.init, Hb, Eseg, Dlog, Lseg, a.final_state, pl.l, h, g, pl.Q, pl.nc,
                       pl.Qp, pl.cps, pl.nseg);
    trace_end(1, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (pl.nseg > 1) {
        const int64_t np4 = (int64_t)N * P / 4;
        const int64_t tot = pl.b * pl.h * np4;
        trace_begin(2, s);
        hipLaunchKernelGGL(k_seg_combine, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, Eseg,
                           Lseg, a.final_state, pl.b * pl.h, h, pl.nseg, np4);
        trace_end(2, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    const int64_t nblk4 = pl.b * pl.nc * pl.h;
    trace_begin(3, s);
    hipLaunchKernelGGL((k_chunk_out<IO, P, N>), dim3((unsigned)nblk4), dim3(256), 0, s, x, Bm, Cm,
                       a.D, lcs, dtp, Hb, Eseg, Dlog, y, pl.l, h, g, pl.Q, pl.nc, pl.Qp, pl.cps,
                       pl.nseg);
    trace_end(3, s);
    return hipGetLastError();
}

}  // namespace ssd
