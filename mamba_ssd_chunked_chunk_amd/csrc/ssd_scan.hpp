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
// Every exponent is <= 0 when A <= 0; the j > i half is removed by a select,
// so no inf * 0 reaches a result.
//
// Launch sequence on one stream:
//   1. k_prep        d and lcs per block (row a1); on the bf16 path also the
//                    fp16 matrix-core copies of B and C
//   2. k_state_pass  chunk states on the matrix cores, serial over chunks
//                    inside a segment; writes the boundary states (rows a2, a3)
//   3. k_seg_combine only when the sequence is cut into several segments:
//                    carries the state across segment ends     (row a3)
//   4. k_chunk_out   per (batch, chunk, head): intra-chunk masked product,
//                    read of the boundary state, skip term     (rows a4, a5)
#pragma once

#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

constexpr int kT = 32;  // rows per block

// True when the matrix-core operand type differs from the io type (bf16 io,
// fp16 operands): B and C are then converted once into the workspace.
template <typename IO>
constexpr bool kOpCopy = !std::is_same<IO, typename Op<IO>::type>::value;

// ----------------------------------------------------------------------------
// 1. Preparation.
//    (a) Time step and per-block cumulative log2 decay, one wave per
//        (batch, head, 64 padded rows), one row per lane:
//          dtp[b, h, R] = d,   lcs[b, h, R] = log2(e) sum_{block start..R} A d
//        over the padded row space (R = c Qp + r); padded rows have d = 0.
//    (b) bf16 io only: B and C converted once to fp16 for the matrix cores of
//        every head of the group (exact inside fp16's normal range).
//    Workgroups [0, na) do (a); the others stride over the pieces of (b).
template <typename IO>
__global__ __launch_bounds__(256) void k_prep(
    const IO *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ dt_bias,
    int softplus, float dt_min, float dt_max, int64_t nbatch, int64_t l, int h, int64_t Q,
    int64_t nc, int64_t Qp, float *__restrict__ lcs, float *__restrict__ dtp, int64_t na,
    const IO *__restrict__ Bm, const IO *__restrict__ Cm, typename Op<IO>::type *__restrict__ Bf,
    typename Op<IO>::type *__restrict__ Cf, int64_t pieces) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((int64_t)blockIdx.x < na) {
        const int64_t lp = nc * Qp, ns = (lp + 63) / 64;
        const int64_t item = (int64_t)blockIdx.x * kWaves + wave;  // (batch, head, slice)
        if (item >= nbatch * h * ns) return;
        const int64_t slice = item % ns, bh = item / ns;
        const int hh = (int)(bh % h);
        const int64_t b = bh / h;
        const int64_t R = slice * 64 + lane;
        const int64_t c = R / Qp, rp = R % Qp, t = c * Q + rp;
        float d = 0.f;
        if (R < lp && rp < Q && t < l)
            d = time_step(to_f32(dt[(b * l + t) * h + hh]), dt_bias ? dt_bias[hh] : 0.f,
                          softplus, dt_min, dt_max);
        float a = A[hh] * kLog2e * d;
        // inclusive scan inside each 32-lane half (a block: Qp and 64 are
        // multiples of kT, so blocks start at lane 0 or 32)
#pragma unroll
        for (int off = 1; off < kT; off <<= 1) {
            const float v = __shfl_up(a, off, kT);
            if ((lane & (kT - 1)) >= off) a += v;
        }
        if (R < lp) {
            lcs[bh * lp + R] = a;
            dtp[bh * lp + R] = d;
        }
        return;
    }
    if constexpr (kOpCopy<IO>) {
        // 8 elements per piece; the pieces of B, then those of C
        const int64_t stride = ((int64_t)gridDim.x - na) * kThreads;
        for (int64_t q = ((int64_t)blockIdx.x - na) * kThreads + threadIdx.x; q < 2 * pieces;
             q += stride) {
            const bool isB = q < pieces;
            const int64_t off = (isB ? q : q - pieces) * 8;
            const Row8v<IO> v = ld_row8((isB ? Bm : Cm) + off);
            Row8v<f16> o;
#pragma unroll
            for (int e = 0; e < 8; e += 2)
                pack2((float)v.e[e], (float)v.e[e + 1], o.e[e], o.e[e + 1]);
            st_row8((isB ? Bf : Cf) + off, o);
        }
    }
}

// ----------------------------------------------------------------------------
// Staging of the state pass: one slab = SLAB blocks of kT rows.  Pieces are
// 8 consecutive elements of one row of x (P / 8 per row) or of B (N / 8 per
// row).  The prefetch only issues loads (row index clamped to row 0 of the
// sequence, which is always readable) and records which pieces are real
// rows; conversions and selects happen in the stage step, so nothing waits
// on a load before it is needed.
template <typename IO, int P, int N, int SLAB> struct SpBuf {
    typedef typename Op<IO>::type OP;
    static constexpr int NPX = SLAB * kT * P / 8, NPB = SLAB * kT * N / 8;
    static constexpr int KX = (NPX + kThreads - 1) / kThreads;
    static constexpr int KB = (NPB + kThreads - 1) / kThreads;
    Row8v<IO> xv[KX];
    Row8v<OP> bv[KB];
    float xl[KX], xd[KX], xe[KX];  // lcs, d of the x piece's row; lcs at its block end
    float lam[SLAB];               // log2 decay of each block of the slab
    uint32_t okx, okb;             // bit k: piece k is a real row
};

template <typename IO, int P, int N, int SLAB>
__device__ __forceinline__ void sp_prefetch(SpBuf<IO, P, N, SLAB> &f, int64_t s0, int64_t sb1,
                                            int64_t nsb, const IO *xb,
                                            const typename Op<IO>::type *Bb,
                                            const float *lcs_bh, const float *dtp_bh, int64_t l,
                                            int64_t Q, int64_t xstride, int64_t bstride, int tid) {
    typedef SpBuf<IO, P, N, SLAB> F;
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
            const int j = q / (N / 8), cc = q % (N / 8), jb = j / T;
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

template <typename IO, int P, int N, int SLAB>
__device__ __forceinline__ void sp_stage(const SpBuf<IO, P, N, SLAB> &f,
                                         typename Op<IO>::type *Xw,
                                         typename Op<IO>::type *Bs, int tid) {
    typedef SpBuf<IO, P, N, SLAB> F;
    typedef typename Op<IO>::type OP;
    constexpr int LDX = P + 16, LDB = N + 16;
#pragma unroll
    for (int k = 0; k < F::KX; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPX % kThreads == 0 || q < F::NPX) {
            const bool ok = (f.okx >> k) & 1;
            const float w = ok ? exp2_fast(f.xe[k] - f.xl[k]) * f.xd[k] : 0.f;
            st_row8(Xw + (q / (P / 8)) * LDX + (q % (P / 8)) * 8, wx_piece(f.xv[k], w));
        }
    }
#pragma unroll
    for (int k = 0; k < F::KB; ++k) {
        const int q = tid + k * kThreads;
        if (F::NPB % kThreads == 0 || q < F::NPB)
            st_row8(Bs + (q / (N / 8)) * LDB + (q % (N / 8)) * 8,
                    keep_or_zero<OP>(f.bv[k], (f.okb >> k) & 1));
    }
}

// ----------------------------------------------------------------------------
// 2. Chunk states and the serial pass over chunks.
//    One workgroup per (batch, segment, head).  The state H (state_dim x
//    head_dim, fp32) lives in MFMA accumulators for the whole segment, its
//    16 x 16 tiles dealt round-robin to the 4 waves.  Slabs of SLAB row
//    blocks are double-buffered in LDS: while one slab is applied, the next
//    is staged and the one after it is being fetched.  Per block:
//        H <- 2^lcs_last H + B^T (w x),  w_j = 2^(lcs_last - lcs_j) d_j,
//    both operands read k-major through transposing LDS loads.  Before the
//    first block of every chunk the state is written out as that chunk's
//    boundary state.  Segment 0 starts from init_state; later segments start
//    from zero and are corrected by k_seg_combine and in k_chunk_out.
template <typename IO, int P, int N>
__global__ __launch_bounds__(256) void k_state_pass(
    const IO *__restrict__ x, const typename Op<IO>::type *__restrict__ Bm,
    const float *__restrict__ lcs, const float *__restrict__ dtp, const float *__restrict__ init,
    float *__restrict__ Hb, float *__restrict__ Eseg, float *__restrict__ Dlog,
    float *__restrict__ Lseg, float *__restrict__ final_state, int64_t l, int h, int g, int64_t Q,
    int64_t nc, int64_t Qp, int64_t cps, int64_t nseg) {
    typedef typename Op<IO>::type OP;
    typedef Mfma<OP> M;
    constexpr int T = kT;
    constexpr int KS = T / M::K;            // MFMA steps per block
    constexpr int SLAB = 2;                 // blocks per slab
    constexpr int SR = SLAB * T;            // rows per slab
    constexpr int LDX = P + 16, LDB = N + 16;
    constexpr int CT = P / 16;
    constexpr int TILES = (N / 16) * CT;
    constexpr int TPW = (TILES + kWaves - 1) / kWaves;
    constexpr int BUF = SR * LDX + SR * LDB;
    __shared__ __attribute__((aligned(16))) OP lds[2 * BUF];  // [w x | B] x 2 buffers

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int hh = (int)(item % h); item /= h;
    const int64_t seg = item % nseg;
    const int64_t b = item / nseg;
    const int gi = hh / (h / g);
    const int64_t nsb = Qp / T;
    const int64_t c0 = seg * cps;
    const int64_t c1 = (c0 + cps < nc) ? c0 + cps : nc;
    const int64_t sb0 = c0 * nsb, sb1 = c1 * nsb;
    const float *lcs_bh = lcs + (b * h + hh) * nc * Qp;
    const float *dtp_bh = dtp + (b * h + hh) * nc * Qp;
    const int64_t NP = (int64_t)N * P;
    const int64_t xs = (int64_t)h * P, bs = (int64_t)g * N;
    const IO *xb = x + (b * l * h + hh) * P;   // row t at xb + t * xs
    const OP *Bb = Bm + (b * l * g + gi) * N;   // row t at Bb + t * bs

    f32x4 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = zero4();
    if (seg == 0 && init) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int ti = wave + kWaves * i;
            if (ti < TILES) {
                const int tr = ti / CT, tc = ti % CT;
                const float *src = init + (b * h + hh) * NP +
                                   (int64_t)(tr * 16 + 4 * (lane >> 4)) * P + tc * 16 +
                                   (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][r] = src[r * P];
            }
        }
    }
    float logdec = 0.f;

    SpBuf<IO, P, N, SLAB> pf;
    const int64_t nslab = (sb1 - sb0 + SLAB - 1) / SLAB;
    float lam_next[SLAB];
    if (nslab > 0) {
        sp_prefetch(pf, sb0, sb1, nsb, xb, Bb, lcs_bh, dtp_bh, l, Q, xs, bs, tid);
#pragma unroll
        for (int jb = 0; jb < SLAB; ++jb) lam_next[jb] = pf.lam[jb];
        sp_stage(pf, lds, lds + SR * LDX, tid);
        if (nslab > 1)
            sp_prefetch(pf, sb0 + SLAB, sb1, nsb, xb, Bb, lcs_bh, dtp_bh, l, Q, xs, bs, tid);
    }
    lds_barrier();
    for (int64_t si = 0; si < nslab; ++si) {
        const int64_t s0 = sb0 + si * SLAB;
        const int nb = (int)((sb1 - s0) < SLAB ? (sb1 - s0) : SLAB);
        float lam[SLAB];
#pragma unroll
        for (int jb = 0; jb < SLAB; ++jb) lam[jb] = lam_next[jb];
        const OP *Xw = lds + (si & 1) * BUF;
        const OP *Bs = Xw + SR * LDX;
        if (si + 1 < nslab) {  // stage the next slab into the other buffer
#pragma unroll
            for (int jb = 0; jb < SLAB; ++jb) lam_next[jb] = pf.lam[jb];
            OP *nx = lds + ((si + 1) & 1) * BUF;
            sp_stage(pf, nx, nx + SR * LDX, tid);
            if (si + 2 < nslab)
                sp_prefetch(pf, s0 + 2 * SLAB, sb1, nsb, xb, Bb, lcs_bh, dtp_bh, l, Q, xs, bs,
                            tid);
        }
#pragma unroll
        for (int jb = 0; jb < SLAB; ++jb) {
            if (jb < nb) {
                const int64_t sb = s0 + jb;
                if (sb % nsb == 0) {  // first block of a chunk: emit the boundary state
                    const int64_t c = sb / nsb;
                    float *dst = Hb + ((b * nc + c) * h + hh) * NP;
#pragma unroll
                    for (int i = 0; i < TPW; ++i) {
                        const int ti = wave + kWaves * i;
                        if (ti < TILES) {
                            const int tr = ti / CT, tc = ti % CT;
                            float *d0 = dst + (int64_t)(tr * 16 + 4 * (lane >> 4)) * P +
                                        tc * 16 + (lane & 15);
#pragma unroll
                            for (int r = 0; r < 4; ++r) d0[r * P] = acc[i][r];
                        }
                    }
                    if (nseg > 1 && tid == 0) Dlog[(b * h + hh) * nc + c] = logdec;
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
                            const int tr = ti / CT, tc = ti % CT;
                            acc[i] = M::mma(frag_kmajor(Bs, LDB, jb * T, q, tr * 16, lane),
                                            frag_kmajor(Xw, LDX, jb * T, q, tc * 16, lane),
                                            acc[i]);
                        }
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
                const int tr = ti / CT, tc = ti % CT;
                float *d0 = out + (int64_t)(tr * 16 + 4 * (lane >> 4)) * P + tc * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) d0[r * P] = acc[i][r];
            }
        }
    }
    if (nseg > 1 && tid == 0) Lseg[(b * h + hh) * nseg + seg] = logdec;
}

// ----------------------------------------------------------------------------
// 3. Segment combine: the state entering segment k (k >= 1) is
//        Hin_{k+1} = 2^L_k Hin_k + E_k,   Hin_1 = E_0,
//    with E_k the state segment k reaches from zero (segment 0: from the
//    initial state) and L_k its total log2 decay.  Hin_k overwrites slot
//    k - 1 of Eseg; the state after the last segment is the final state.
//    One thread per 4 consecutive state elements of one (batch, head); the
//    segment states are loaded in groups of 8 before any of them is used.
static __global__ __launch_bounds__(256) void k_seg_combine(float *__restrict__ Eseg,
                                                            const float *__restrict__ Lseg,
                                                            float *__restrict__ final_state,
                                                            int64_t bh, int h, int64_t nseg,
                                                            int64_t np4) {
    constexpr int G8 = 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= bh * np4) return;
    const int64_t pair = idx / np4, e4 = idx % np4;
    const int64_t b = pair / h, hh = pair % h;
    f32x4 *E = reinterpret_cast<f32x4 *>(Eseg) + (b * nseg * h + hh) * np4 + e4;
    const int64_t stride = (int64_t)h * np4;  // from one segment slot to the next
    f32x4 H = E[0];
    for (int64_t k0 = 1; k0 < nseg; k0 += G8) {
        f32x4 Ek[G8];
        float Lk[G8];
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int64_t k = k0 + u < nseg ? k0 + u : nseg - 1;
            Ek[u] = E[k * stride];
            Lk[u] = Lseg[pair * nseg + k];
        }
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            if (k0 + u < nseg) {
                E[(k0 + u - 1) * stride] = H;      // Hin_k, k = k0 + u
                H = exp2_fast(Lk[u]) * H + Ek[u];  // Hin_{k+1}
            }
        }
    }
    if (final_state) reinterpret_cast<f32x4 *>(final_state)[pair * np4 + e4] = H;
}

// ----------------------------------------------------------------------------
// Staging of the chunk output: one block of kT rows.  Pieces are 8
// consecutive elements of one row of C and of B (same row and columns, N / 8
// per row) or of x (P / 8 per row).  As in the state pass, the prefetch only
// issues loads and records which pieces are real rows.
template <typename IO, int P, int N, int NT> struct CoBuf {
    typedef typename Op<IO>::type OP;
    static constexpr int NPC = kT * N / 8, NPX = kT * P / 8;
    static constexpr int KC = (NPC + NT - 1) / NT;
    static constexpr int KX = (NPX + NT - 1) / NT;
    Row8v<OP> cv[KC], bv[KC];
    Row8v<IO> xv[KX];
    float xl[KX], xd[KX];  // lcs and d of the x piece's row
    float last, ls, ds;    // lcs at the block end; lcs and d of row tid (tid < kT)
    uint32_t okc, okx;
};

template <typename IO, int P, int N, int NT>
__device__ __forceinline__ void co_prefetch(CoBuf<IO, P, N, NT> &f, int s, const IO *xb,
                                            const typename Op<IO>::type *Bb,
                                            const typename Op<IO>::type *Cb, const float *lcs_c,
                                            const float *dtp_c, int64_t t0, int64_t l, int64_t Q,
                                            int64_t xstride, int64_t bstride, int tid) {
    typedef CoBuf<IO, P, N, NT> F;
    constexpr int T = kT;
    const int64_t rpb = (int64_t)s * T;
    f.okc = 0;
    f.okx = 0;
#pragma unroll
    for (int k = 0; k < F::KC; ++k) {
        const int q = tid + k * NT;
        if (F::NPC % NT == 0 || q < F::NPC) {
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
        const int q = tid + k * NT;
        if (F::NPX % NT == 0 || q < F::NPX) {
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

template <typename IO, int P, int N, int NT>
__device__ __forceinline__ void co_stage(const CoBuf<IO, P, N, NT> &f, typename Op<IO>::type *Cs,
                                         typename Op<IO>::type *Bs, typename Op<IO>::type *Xs,
                                         typename Op<IO>::type *Xw, float *lcs_s, float *lcsd_s,
                                         int tid) {
    typedef CoBuf<IO, P, N, NT> F;
    typedef typename Op<IO>::type OP;
    constexpr int LDN = N + Mfma<OP>::PAD, LDX = P + 16;
#pragma unroll
    for (int k = 0; k < F::KC; ++k) {
        const int q = tid + k * NT;
        if (F::NPC % NT == 0 || q < F::NPC) {
            const int o = (q / (N / 8)) * LDN + (q % (N / 8)) * 8;
            const bool ok = (f.okc >> k) & 1;
            st_row8(Cs + o, keep_or_zero<OP>(f.cv[k], ok));
            st_row8(Bs + o, keep_or_zero<OP>(f.bv[k], ok));
        }
    }
#pragma unroll
    for (int k = 0; k < F::KX; ++k) {
        const int q = tid + k * NT;
        if (F::NPX % NT == 0 || q < F::NPX) {
            const int o = (q / (P / 8)) * LDX + (q % (P / 8)) * 8;
            const bool ok = (f.okx >> k) & 1;
            const float w = ok ? exp2_fast(f.last - f.xl[k]) * f.xd[k] : 0.f;
            Row8v<OP> xo, wo;
            x_pieces(f.xv[k], w, ok, xo, wo);
            st_row8(Xs + o, xo);
            st_row8(Xw + o, wo);
        }
    }
    if (tid < kT) {
        lcs_s[tid] = f.ls;
        // the score weight 2^(lcs_i - lcs_j) d_j is taken as 2^(lcs_i - lcsd_j)
        // with lcsd_j = lcs_j - log2 d_j; d = 0 gives +inf and weight 0
        lcsd_s[tid] = f.ls - __builtin_amdgcn_logf(f.ds);
    }
}

// ----------------------------------------------------------------------------
// 4. Chunk output.  One workgroup per (batch, chunk, head), W = min(4,
//    head_dim / 16) waves.  Wave w owns the head_dim column tiles
//    pt = w, w + W, ... of everything it produces: its columns of the running
//    state H (all state_dim rows) stay in MFMA accumulators across the
//    chunk's blocks and feed the output product straight from registers, and
//    it computes y^T for those columns, so that each lane holds 4
//    consecutive head_dim values of one row (one vector store).  Per block,
//    with C, B, x and w x double-buffered in LDS and the block after next
//    already being fetched:
//      G^T = B C^T on the 3 causal 16 x 16 tiles, and
//      P_ij = G_ij 2^(lcs_i - lcs_j) d_j (j <= i), in registers;
//      y^T = 2^lcs_i (H^T C^T) + x^T P^T + D x^T, written to y;
//      H <- 2^lcs_last H + B^T (w x)  (except after the last block).
//    One workgroup barrier per block.
template <int P> struct CoShape {
    static constexpr int W = P >= 64 ? 4 : P / 16;  // waves
    static constexpr int NT = 64 * W;               // threads
};

template <typename IO, int P, int N>
__global__ __launch_bounds__(CoShape<P>::NT) void k_chunk_out(
    const IO *__restrict__ x, const typename Op<IO>::type *__restrict__ Bm,
    const typename Op<IO>::type *__restrict__ Cm, const float *__restrict__ D,
    const float *__restrict__ lcs, const float *__restrict__ dtp, const float *__restrict__ Hb,
    const float *__restrict__ Hin, const float *__restrict__ Dlog, IO *__restrict__ y,
    int64_t l, int h, int g, int64_t Q, int64_t nc, int64_t Qp, int64_t cps, int64_t nseg) {
    typedef typename Op<IO>::type OP;
    typedef Mfma<OP> M;
    constexpr int W = CoShape<P>::W, NT = CoShape<P>::NT;
    constexpr int T = kT;
    constexpr int KS = T / M::K;          // MFMA steps over 32 contraction indices
    constexpr int NS = N / M::K;          // MFMA steps over the state index
    constexpr int NB = N / 32;            // 32-blocks of the state index
    constexpr int LDN = N + M::PAD;       // [row][n]: C, B
    constexpr int LDX = P + 16;           // [row][p]: x, w x
    constexpr int CT = P / 16;            // head_dim column tiles
    constexpr int CPW = CT / W;           // column tiles per wave
    constexpr int RT = N / 16;            // state row tiles
    constexpr int BUF = 2 * T * LDN + 2 * T * LDX;
    __shared__ __attribute__((aligned(16))) OP lds[2 * BUF];  // [C | B | x | w x] x 2
    __shared__ float lcs_s[2][T];
    __shared__ float lcsd_s[2][T];

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
    const int64_t xs = (int64_t)h * P, bs = (int64_t)g * N, t0 = c * Q;
    const IO *xb = x + (b * l * h + hh) * P;   // row t at xb + t * xs
    const OP *Bb = Bm + (b * l * g + gi) * N;   // row t at Bb + t * bs
    const OP *Cb = Cm + (b * l * g + gi) * N;
    IO *yb = y + (b * l * h + hh) * P;

    CoBuf<IO, P, N, NT> pf;
    co_prefetch(pf, 0, xb, Bb, Cb, lcs_c, dtp_c, t0, l, Q, xs, bs, tid);

    // ---- the wave's state columns entering the chunk (all loads issued first)
    f32x4 accH[CPW][RT];
    {
        const float *hb = Hb + ((b * nc + c) * h + hh) * NP;
#pragma unroll
        for (int u = 0; u < CPW; ++u)
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) {
                const int64_t off = (int64_t)(tr * 16 + 4 * lg) * P + (wave + W * u) * 16 + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) accH[u][tr][r] = hb[off + r * P];
            }
        if (seg > 0) {
            const float *hin = Hin + ((b * nseg + seg - 1) * h + hh) * NP;
            f32x4 iv[CPW][RT];
#pragma unroll
            for (int u = 0; u < CPW; ++u)
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) {
                    const int64_t off =
                        (int64_t)(tr * 16 + 4 * lg) * P + (wave + W * u) * 16 + li;
#pragma unroll
                    for (int r = 0; r < 4; ++r) iv[u][tr][r] = hin[off + r * P];
                }
            const float corr = exp2_fast(Dlog[(b * h + hh) * nc + c]);
#pragma unroll
            for (int u = 0; u < CPW; ++u)
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) accH[u][tr] += corr * iv[u][tr];
        }
    }

    co_stage(pf, lds, lds + T * LDN, lds + 2 * T * LDN, lds + 2 * T * LDN + T * LDX, lcs_s[0],
             lcsd_s[0], tid);
    if (nblk > 1) co_prefetch(pf, 1, xb, Bb, Cb, lcs_c, dtp_c, t0, l, Q, xs, bs, tid);
    lds_barrier();

    for (int s = 0; s < nblk; ++s) {
        const int cur = s & 1;
        const OP *Cs = lds + cur * BUF;
        const OP *Bs = Cs + T * LDN;
        const OP *Xs = Bs + T * LDN;
        const OP *Xw = Xs + T * LDX;
        const float *ls = lcs_s[cur];
        const float *lsd = lcsd_s[cur];
        if (s + 1 < nblk) {  // stage the next block into the other buffer
            OP *nC = lds + (cur ^ 1) * BUF;
            co_stage(pf, nC, nC + T * LDN, nC + 2 * T * LDN, nC + 2 * T * LDN + T * LDX,
                     lcs_s[cur ^ 1], lcsd_s[cur ^ 1], tid);
            if (s + 2 < nblk)
                co_prefetch(pf, s + 2, xb, Bb, Cb, lcs_c, dtp_c, t0, l, Q, xs, bs, tid);
        }

        // ---- masked, decayed scores: G^T tiles (jt, it), jt <= it.
        //      pv[it][jt] element r: j = 16 jt + 4 lg + r, i = 16 it + li
        f32x4 pv[2][2];
        pv[0][1] = zero4();
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = it * 16 + li;
            const float lci = ls[i];
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
                f32x4 gacc = zero4();
#pragma unroll
                for (int ks = 0; ks < NS; ++ks)
                    gacc = M::mma(lds_frag(Bs, LDN, jt * 16, ks * M::K, lane),
                                  lds_frag(Cs, LDN, it * 16, ks * M::K, lane), gacc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = jt * 16 + 4 * lg + r;
                    pv[it][jt][r] = (j <= i) ? gacc[r] * exp2_fast(lci - lsd[j]) : 0.f;
                }
            }
        }

        // ---- y^T tiles of the wave's columns: element r of lane l is
        //      (p = 16 pt + 4 lg + r, i = 16 it + li)
        const int64_t rpb = (int64_t)s * T;
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            const int pt = wave + W * u;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int i = it * 16 + li;
                f32x4 ya = zero4();
#pragma unroll
                for (int m = 0; m < NB; ++m)
#pragma unroll
                    for (int q = 0; q < KS; ++q)
                        ya = M::mma(frag_from_acc<OP>(accH[u][2 * m], accH[u][2 * m + 1], q),
                                    frag_rows_kconv(Cs, LDN, it * 16, 32 * m, q, lane), ya);
                ya *= exp2_fast(ls[i]);
#pragma unroll
                for (int q = 0; q < KS; ++q)
                    ya = M::mma(frag_kmajor(Xs, LDX, 0, q, pt * 16, lane),
                                frag_from_acc<OP>(pv[it][0], pv[it][1], q), ya);
                const f32x4 xv = lds_load4(Xs + i * LDX + pt * 16 + 4 * lg);
                const int64_t rp = rpb + i;
                if (rp < rows) store4(yb + (t0 + rp) * xs + pt * 16 + 4 * lg, ya + Dh * xv);
            }
        }

        // ---- carry the state to the next block of the chunk
        if (s + 1 < nblk) {
            const float decay = exp2_fast(ls[T - 1]);
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const int pt = wave + W * u;
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) {
                    accH[u][tr] *= decay;
#pragma unroll
                    for (int q = 0; q < KS; ++q)
                        accH[u][tr] = M::mma(frag_kmajor(Bs, LDN, 0, q, tr * 16, lane),
                                             frag_kmajor(Xw, LDX, 0, q, pt * 16, lane),
                                             accH[u][tr]);
                }
            }
        }
        lds_barrier();  // this block's buffer is free; the next one is staged
    }
}

// ----------------------------------------------------------------------------
template <typename IO, int P, int N>
hipError_t launch_scan(const ScanPlan &pl, const ScanArgs &a, hipStream_t s) {
    typedef typename Op<IO>::type OP;
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
    // matrix-core operands B and C: the fp16 copies, or the fp32 inputs
    OP *Bf = reinterpret_cast<OP *>(a.ws + pl.off_bf);
    OP *Cf = reinterpret_cast<OP *>(a.ws + pl.off_cf);
    const OP *Bop = kOpCopy<IO> ? Bf : reinterpret_cast<const OP *>(Bm);
    const OP *Cop = kOpCopy<IO> ? Cf : reinterpret_cast<const OP *>(Cm);

    const int64_t ns = (pl.lp + 63) / 64;
    const int64_t na = (pl.b * pl.h * ns + kWaves - 1) / kWaves;
    const int64_t pieces = pl.b * pl.l * pl.g * pl.n / 8;
    int64_t ncopy = 0;
    if (kOpCopy<IO>) {
        ncopy = (2 * pieces + kThreads - 1) / kThreads;
        if (ncopy > 2048) ncopy = 2048;
    }
    trace_begin(0, s);
    hipLaunchKernelGGL(k_prep<IO>, dim3((unsigned)(na + ncopy)), dim3(kThreads), 0, s, dt, a.A,
                       a.dt_bias, a.softplus, a.dt_min, a.dt_max, pl.b, pl.l, h, pl.Q, pl.nc,
                       pl.Qp, lcs, dtp, na, Bm, Cm, Bf, Cf, pieces);
    trace_end(0, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    trace_begin(1, s);
    hipLaunchKernelGGL((k_state_pass<IO, P, N>), dim3((unsigned)(pl.b * pl.nseg * pl.h)),
                       dim3(kThreads), 0, s, x, Bop, lcs, dtp, a.init, Hb, Eseg, Dlog, Lseg,
                       a.final_state, pl.l, h, g, pl.Q, pl.nc, pl.Qp, pl.cps, pl.nseg);
    trace_end(1, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (pl.nseg > 1) {
        const int64_t np4 = (int64_t)N * P / 4;
        const int64_t tot = pl.b * pl.h * np4;
        trace_begin(2, s);
        hipLaunchKernelGGL(k_seg_combine, dim3((unsigned)((tot + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, s, Eseg, Lseg, a.final_state, pl.b * pl.h, h,
                           pl.nseg, np4);
        trace_end(2, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    trace_begin(3, s);
    hipLaunchKernelGGL((k_chunk_out<IO, P, N>), dim3((unsigned)(pl.b * pl.nc * pl.h)),
                       dim3(CoShape<P>::NT), 0, s, x, Bop, Cop, a.D, lcs, dtp, Hb, Eseg, Dlog, y,
                       pl.l, h, g, pl.Q, pl.nc, pl.Qp, pl.cps, pl.nseg);
    trace_end(3, s);
    return hipGetLastError();
}

}  // namespace ssd
