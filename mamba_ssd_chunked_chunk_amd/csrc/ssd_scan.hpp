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
// boundary; lcs_i is the cumulative log2 decay inside a block (inclusive),
// lam_K the total of block K.  With Lambda_i the cumulative log2 decay from
// the chunk start (a sum of block totals plus one lcs) and H_c the state
// entering chunk c:
//   S_c     = sum_j 2^(Lambda_last - Lambda_j) d_j B_j x_j^T   (chunk state)
//   H_{c+1} = 2^(Lambda_last) H_c + S_c                        (state scan)
//   y_i     = sum_{j<=i} (C_i . B_j) 2^(Lambda_i - Lambda_j) d_j x_j
//             + 2^Lambda_i C_i^T H_c + D x_i                    (chunk output)
// Every exponent is <= 0 when A <= 0; the j > i half is removed by a select,
// so no inf * 0 reaches a result.
//
// Launch sequence on one stream:
//   1. k_chunk_state  per row: d, lcs and the state weights; every chunk's
//                     state from zero and its total decay, all chunks in
//                     parallel, on the matrix cores
//   2. k_state_scan   the serial pass over chunks: boundary states (as the
//                     read-out's matrix-core operand) and the final state
//   3. k_chunk_out    per (batch, chunk, heads): intra-chunk masked product,
//                     read-out of the boundary state, skip term
#pragma once

#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

constexpr int kT = 32;  // rows per block

// Heads of one group handled by one workgroup of the state pass and of the
// chunk output when the group size allows it (see group_heads in the plan):
// B and C are staged once for all of them.
template <int P> constexpr int kGroupHeads = P >= 64 ? 128 / P : 4;

// ----------------------------------------------------------------------------
// An io piece of 8 elements -> matrix-core operand piece (bf16 -> fp16:
// exact inside fp16's normal range).
__device__ __forceinline__ Row8v<f16> op_piece(const Row8v<bf16> &v) {
    Row8v<f16> o;
#pragma unroll
    for (int e = 0; e < 8; e += 2) pack2((float)v.e[e], (float)v.e[e + 1], o.e[e], o.e[e + 1]);
    return o;
}
__device__ __forceinline__ Row8v<float> op_piece(const Row8v<float> &v) { return v; }

// ----------------------------------------------------------------------------
// 1. Chunk states, with the per-row preparation folded in.  One workgroup
//    per (batch, chunk, HPW consecutive heads of one group); WPH = max(1,
//    head_dim / 32) waves per head, each owning 32 (or head_dim) head_dim
//    columns of its head's chunk state (state_dim x head_dim, fp32) in MFMA
//    accumulators.
//    The chunk goes in spans of up to SPAN = 8 blocks (256 rows).  At the
//    start of a span the workgroup turns the span's raw time steps into the
//    per-row values of each head (one row per thread, a block per 32 lanes):
//        d_r   = clamp(softplus(dt_r + bias))  (0 on padded rows),
//        lcs_r = log2(e) sum_{block start..r} A d   (inclusive),
//        w_r   = 2^(lcs_last - lcs_r) d_r   (weight of row r in the state at
//                the end of its block),
//    writes them out for the chunk output and keeps in LDS the weight of
//    every row in the state at the span's end,
//        v_r = w_r 2^(lam_{J+1} + ... + lam_{span's last block})
//    (row r in block J, every factor <= 1).  The state then decays once per
//    span, S <- 2^L S (L the span's log2 decay), and every block adds
//    S += B^T (v x) with x weighted as it is staged, so a block costs its
//    staging and its products only.  Blocks are fetched two ahead into
//    registers (B once for all heads, x per head) and staged through one
//    LDS buffer; both operands are read k-major through transposing LDS
//    loads.  The state is written transposed ([head_dim][state_dim], one
//    16-byte store per lane and tile) with the chunk's total log2 decay.
template <typename IO, int P, int N, int HPW> struct Sp {
    typedef typename Op<IO>::type OP;
    typedef Mfma<OP> M;
    static constexpr int T = kT;
    static constexpr int SPAN = 8, SPR = SPAN * T;    // blocks and rows per span
    static constexpr int WPH = P >= 64 ? P / 32 : 1;  // waves per head
    static constexpr int PW = P / WPH;                // head_dim columns per wave
    static constexpr int CPW = PW / 16;               // column tiles per wave
    static constexpr int W = HPW * WPH, NT = 64 * W;  // waves, threads
    static constexpr int RT = N / 16;                 // state row tiles
    static constexpr int TPW = CPW * RT;              // tiles per wave
    static constexpr int KS = T / M::K;               // MFMA steps per block
    static constexpr int LDX = P + 16, LDB = N + 16;  // padded rows (transposing reads)
    static constexpr int XS = T * LDX;                // one head's staged v x
    static constexpr int BUF = T * LDB + HPW * XS;    // [B | v x of each head]
    static constexpr int NPB = T * N / 8, NPX = HPW * T * P / 8;  // pieces of 8
    static constexpr int KB = (NPB + NT - 1) / NT, KX = (NPX + NT - 1) / NT;
    static constexpr int NPASS = HPW * SPR / NT;      // span rows per thread
    static_assert(NPASS * NT == HPW * SPR && NT % 64 == 0, "span rows in whole waves");
};

// Per-row weights of the current span, per head (LDS).
template <int HPW> struct SpSpan {
    float v[HPW][8 * kT];  // weight in the state at the span's end
    float lam[HPW][8];     // log2 decay of each block of the span
};

// Register prefetch of one block.  Loads go through buffer resources that
// end at the chunk's last valid row (zeros beyond); a block past the chunk's
// end issues the same loads with empty resources.
template <typename IO, int P, int N, int HPW> struct SpBuf {
    typedef Sp<IO, P, N, HPW> K;
    Row8v<IO> bv[K::KB];
    Row8v<IO> xv[K::KX];
};

// Addressing and time-step processing of one workgroup's chunk.
template <typename IO, int HPW> struct SpPtrs {
    const IO *x;             // row 0 of the sequence, first head of the workgroup
    const IO *B;             // row 0 of the sequence, the group
    const IO *dt;            // row 0 of the sequence, first head of the workgroup
    float *lcs, *dtp, *wgt;  // (batch, first head) padded row arrays, written
    int *sgr;                // packed sequences: each row's last reset in its block, or -1
    float a2[HPW], bias[HPW];  // A log2(e) and dt_bias of the workgroup's heads
    int softplus;
    float dt_min, dt_max;
    int64_t xs, bs;          // row strides (elements) of x and of B
    int64_t l, Q, hrow;      // sequence length, chunk, elements from one head's row arrays to the next
    int h;                   // heads (row stride of dt)
    int64_t Qp;              // padded rows per chunk
    const int32_t *seq;      // row 0 of the sequence's document indices (packed sequences)
    // fp32 io only, or NULL: every row's weight and log2 decay given directly
    // (row 0 of the sequence, first head of the workgroup; rows h apart) in
    // place of the time step (the scans of the gradient pass)
    const float *lw, *la;
};

template <typename IO, int P, int N, int HPW>
__device__ __forceinline__ void sp_prefetch(SpBuf<IO, P, N, HPW> &f, int64_t c, int blk,
                                            bool live, const SpPtrs<IO, HPW> &sp, int tid) {
    typedef Sp<IO, P, N, HPW> K;
    constexpr int T = kT;
    const int64_t row0 = c * sp.Q + (int64_t)blk * T;                  // sequence row
    const int64_t cend = (c + 1) * sp.Q < sp.l ? (c + 1) * sp.Q : sp.l;  // end of the chunk
    int64_t valid = live ? cend - row0 : 0;
    valid = valid < 0 ? 0 : (valid > T ? T : valid);
    const int64_t rr0 = valid > 0 ? row0 : 0;
    const Rsrc rx = make_rsrc(sp.x + rr0 * sp.xs, valid * sp.xs * (int64_t)sizeof(IO));
    const Rsrc rb = make_rsrc(sp.B + rr0 * sp.bs, valid * sp.bs * (int64_t)sizeof(IO));
#pragma unroll
    for (int k = 0; k < K::KB; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPB % K::NT == 0 || q < K::NPB) {
            const int j = q / (N / 8), cc = q % (N / 8);
            f.bv[k] = buf_row8<IO>(rb, (uint32_t)(j * sp.bs + cc * 8) * (uint32_t)sizeof(IO));
        }
    }
#pragma unroll
    for (int k = 0; k < K::KX; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPX % K::NT == 0 || q < K::NPX) {
            const int hs = q / (T * P / 8), qq = q % (T * P / 8);
            const int j = qq / (P / 8), cc = qq % (P / 8);
            f.xv[k] = buf_row8<IO>(rx, (uint32_t)(j * sp.xs + hs * P + cc * 8) *
                                           (uint32_t)sizeof(IO));
        }
    }
}

// The raw time steps of the span starting at block blk0, one row of one head
// per thread and pass.
template <typename IO, int P, int N, int HPW, bool SEQ>
__device__ __forceinline__ void sp_dt_load(float *dtv, float *dav, int *rst, int64_t c,
                                           int blk0, const SpPtrs<IO, HPW> &sp, int tid) {
    typedef Sp<IO, P, N, HPW> K;
    constexpr int T = kT;
    const int64_t cend = (c + 1) * sp.Q < sp.l ? (c + 1) * sp.Q : sp.l;
#pragma unroll
    for (int ps = 0; ps < K::NPASS; ++ps) {
        const int idx = ps * K::NT + tid;
        const int hs = idx / K::SPR, r = idx % K::SPR;
        const int64_t row = c * sp.Q + (int64_t)blk0 * T + r;
        if (sizeof(IO) == 4 && sp.lw) {
            dtv[ps] = row < cend ? sp.lw[row * sp.h + hs] : 0.f;
            dav[ps] = row < cend ? sp.la[row * sp.h + hs] : 0.f;
        } else {
            dtv[ps] = row < cend ? to_f32(sp.dt[row * sp.h + hs]) : 0.f;
        }
        // packed sequences: a row whose document index differs from the
        // previous row's starts from a zero state
        if constexpr (SEQ)
            rst[ps] = (row < cend && row > 0) ? (sp.seq[row] != sp.seq[row - 1]) : 0;
    }
}

// The per-row values of the span starting at block blk0 (see above) from
// its raw time steps; ends with the span's weights visible to the whole
// workgroup.
template <typename IO, int P, int N, int HPW, bool SEQ>
__device__ __forceinline__ void sp_span(SpSpan<HPW> &sv, const float *dtv, const float *dav,
                                        const int *rst, int64_t c, int blk0,
                                        const SpPtrs<IO, HPW> &sp, int tid) {
    typedef Sp<IO, P, N, HPW> K;
    constexpr int T = kT;
    const int64_t cend = (c + 1) * sp.Q < sp.l ? (c + 1) * sp.Q : sp.l;
#pragma unroll
    for (int ps = 0; ps < K::NPASS; ++ps) {
        const int idx = ps * K::NT + tid;
        const int hs = idx / K::SPR, r = idx % K::SPR;
        const int64_t row = c * sp.Q + (int64_t)blk0 * T + r;
        // the head's constants, selected without indexing (registers)
        float bias = sp.bias[0], a2 = sp.a2[0];
#pragma unroll
        for (int k = 1; k < HPW; ++k) {
            bias = hs == k ? sp.bias[k] : bias;
            a2 = hs == k ? sp.a2[k] : a2;
        }
        float d, a;
        if (sizeof(IO) == 4 && sp.lw) {
            d = row < cend ? dtv[ps] : 0.f;
            a = row < cend ? dav[ps] : 0.f;
        } else {
            d = row < cend ? time_step(dtv[ps], bias, sp.softplus, sp.dt_min, sp.dt_max) : 0.f;
            a = a2 * d;
        }
        // inclusive scan inside each 32-lane group (one block each)
#pragma unroll
        for (int off = 1; off < T; off <<= 1) {
            const float v = __shfl_up(a, off, T);
            if ((r & (T - 1)) >= off) a += v;
        }
        const float last = __shfl(a, T - 1, T);
        float w = exp2_fast(last - a) * d;
        float lam = last;  // the block's log2 decay
        int seg = -1;      // the last reset at or before this row in its block
        if constexpr (SEQ) {
            // resets in this block (its 32 lanes): rows before the last one
            // do not reach the block's end, and nothing crosses the block
            const uint32_t m = (uint32_t)(__ballot(rst[ps] != 0) >> (tid & 32));
            if (m) {
                if ((r & (T - 1)) < 31 - __builtin_clz(m)) w = 0.f;
                lam = -INFINITY;
            }
            const uint32_t mr = m & ((2u << (r & (T - 1))) - 1u);
            seg = mr ? 31 - __builtin_clz(mr) : -1;
        }
        const int64_t R = (int64_t)blk0 * T + r;  // padded row inside the chunk
        if (R < sp.Qp) {
            const int64_t idx2 = hs * sp.hrow + c * sp.Qp + R;
            sp.lcs[idx2] = a;
            sp.dtp[idx2] = d;
            sp.wgt[idx2] = w;
            if constexpr (SEQ) sp.sgr[idx2] = seg;
        }
        sv.v[hs][r] = w;
        if ((r & (T - 1)) == T - 1) sv.lam[hs][r / T] = lam;
    }
    lds_barrier();
#pragma unroll
    for (int ps = 0; ps < K::NPASS; ++ps) {
        const int idx = ps * K::NT + tid;
        const int hs = idx / K::SPR, r = idx % K::SPR;
        float sfx = 0.f;  // decay of the span's later blocks
#pragma unroll
        for (int k = 0; k < K::SPAN; ++k) sfx += k > r / T ? sv.lam[hs][k] : 0.f;
        sv.v[hs][r] *= exp2_fast(sfx);
    }
    lds_barrier();
}

// v x piece of 8 elements as operands.
__device__ __forceinline__ Row8v<f16> vx_piece(const Row8v<bf16> &x, float v) {
    Row8v<f16> o;
#pragma unroll
    for (int e = 0; e < 8; e += 2) pack2((float)x.e[e] * v, (float)x.e[e + 1] * v, o.e[e], o.e[e + 1]);
    return o;
}
__device__ __forceinline__ Row8v<float> vx_piece(const Row8v<float> &x, float v) {
    Row8v<float> o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o.e[e] = x.e[e] * v;
    return o;
}

// Stages block jb of the span: B as operand, x weighted by v.
template <typename IO, int P, int N, int HPW>
__device__ __forceinline__ void sp_stage(const SpBuf<IO, P, N, HPW> &f, typename Op<IO>::type *buf,
                                         const SpSpan<HPW> &sv, int jb, int tid) {
    typedef Sp<IO, P, N, HPW> K;
    typedef typename K::OP OP;
    constexpr int T = kT;
    OP *Bs = buf, *Xs = buf + T * K::LDB;
#pragma unroll
    for (int k = 0; k < K::KB; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPB % K::NT == 0 || q < K::NPB)
            st_row8(Bs + (q / (N / 8)) * K::LDB + (q % (N / 8)) * 8, op_piece(f.bv[k]));
    }
#pragma unroll
    for (int k = 0; k < K::KX; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPX % K::NT == 0 || q < K::NPX) {
            const int hs = q / (T * P / 8), qq = q % (T * P / 8);
            const int j = qq / (P / 8);
            st_row8(Xs + hs * K::XS + j * K::LDX + (qq % (P / 8)) * 8,
                    vx_piece(f.xv[k], sv.v[hs][jb * T + j]));
        }
    }
}

// Transposed store of the wave's state tiles ([head_dim][state_dim]).
template <typename IO, int P, int N, int HPW>
__device__ __forceinline__ void sp_store_t(float *dst, const f32x4 *acc, int c0, int lane) {
    typedef Sp<IO, P, N, HPW> K;
#pragma unroll
    for (int u = 0; u < K::CPW; ++u)
#pragma unroll
        for (int tr = 0; tr < K::RT; ++tr)
            *reinterpret_cast<f32x4 *>(dst + (c0 + 16 * u + (lane & 15)) * N + tr * 16 +
                                       4 * (lane >> 4)) = acc[u * K::RT + tr];
}

// The same tiles as fp16 times inv (an exact power of two), 8 bytes per 4.
template <typename IO, int P, int N, int HPW>
__device__ __forceinline__ void sp_store_t16(f16 *dst, const f32x4 *acc, float inv, int c0,
                                             int lane) {
    typedef Sp<IO, P, N, HPW> K;
#pragma unroll
    for (int u = 0; u < K::CPW; ++u)
#pragma unroll
        for (int tr = 0; tr < K::RT; ++tr) {
            const f32x4 v = acc[u * K::RT + tr] * inv;
            *reinterpret_cast<f16x4 *>(dst + (c0 + 16 * u + (lane & 15)) * N + tr * 16 +
                                       4 * (lane >> 4)) =
                f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
        }
}

// Adds the staged block to the wave's tiles: S += B^T (v x).
template <typename IO, int P, int N, int HPW>
__device__ __forceinline__ void sp_apply(f32x4 *acc, const typename Op<IO>::type *buf, int hs,
                                         int c0, int lane) {
    typedef Sp<IO, P, N, HPW> K;
    typedef typename K::M M;
    constexpr int KS = K::KS;
    const auto *Bs = buf;
    const auto *Xs = buf + kT * K::LDB + hs * K::XS;
#pragma unroll
    for (int q = 0; q < KS; ++q) {
        typename Mfma<typename K::OP>::frag xf[K::CPW];
#pragma unroll
        for (int u = 0; u < K::CPW; ++u) xf[u] = frag_kmajor(Xs, K::LDX, 0, q, c0 + 16 * u, lane);
#pragma unroll
        for (int tr = 0; tr < K::RT; ++tr) {
            const auto bt = frag_kmajor(Bs, K::LDB, 0, q, tr * 16, lane);
#pragma unroll
            for (int u = 0; u < K::CPW; ++u)
                acc[u * K::RT + tr] = M::mma(bt, xf[u], acc[u * K::RT + tr]);
        }
    }
}

// Workgroups per compute unit the bf16 chunk-state pass is compiled for:
// three (at most 168 VGPRs), except for packed-sequence instances whose
// reset masks would then spill (one-head workgroups, and four heads of
// head_dim 32 with state_dim 128), which get two.
template <int P, int N, int HPW, bool SEQ> constexpr int cs_waves() {
    return SEQ && (HPW == 1 || (P == 32 && N == 128)) ? 2 : 3;
}

template <typename IO, int P, int N, int HPW, bool SEQ>
__global__ __launch_bounds__((Sp<IO, P, N, HPW>::NT),
                             (sizeof(IO) == 2 ? cs_waves<P, N, HPW, SEQ>() : 1)) void k_chunk_state(
    const IO *__restrict__ x, const IO *__restrict__ Bm, const IO *__restrict__ dt,
    const float *__restrict__ A, const float *__restrict__ dt_bias, int softplus, float dt_min,
    float dt_max, float *__restrict__ lcs, float *__restrict__ dtp, float *__restrict__ wgt,
    float *__restrict__ St, float *__restrict__ Lam, float *__restrict__ Scl, int64_t l, int h,
    int g, int64_t Q, int64_t nc, int64_t Qp, int keep_last, const int32_t *__restrict__ seq,
    int *__restrict__ sgr, const float *__restrict__ lw, const float *__restrict__ la) {
    typedef Sp<IO, P, N, HPW> K;
    typedef typename K::OP OP;
    constexpr int T = kT, SPAN = K::SPAN, TPW = K::TPW;
    __shared__ __attribute__((aligned(16))) OP lds0[K::BUF];
    __shared__ __attribute__((aligned(16))) OP lds1[K::BUF];
    __shared__ __attribute__((aligned(16))) SpSpan<HPW> span;
    __shared__ float wmax[K::W];

    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int hq = (int)(item % (h / HPW)); item /= (h / HPW);
    const int64_t c = item % nc;
    const int64_t b = item / nc;
    const int hh0 = hq * HPW;
    const int gi = hh0 / (h / g);
    const int hs = wave / K::WPH;                  // this wave's head slot
    const int hh = hh0 + hs;
    const int c0 = (wave % K::WPH) * K::PW;        // this wave's first column
    const int nsb = (int)(Qp / T);
    const int64_t NP = (int64_t)N * P;
    SpPtrs<IO, HPW> sp;
    sp.xs = (int64_t)h * P;
    sp.bs = (int64_t)g * N;
    sp.x = x + (b * l * h + hh0) * P;
    sp.B = Bm + (b * l * g + gi) * N;
    sp.dt = dt + b * l * h + hh0;
    sp.seq = SEQ ? seq + b * l : nullptr;
    sp.lw = lw ? lw + b * l * h + hh0 : nullptr;
    sp.la = la ? la + b * l * h + hh0 : nullptr;
    sp.lcs = lcs + (b * h + hh0) * nc * Qp;
    sp.dtp = dtp + (b * h + hh0) * nc * Qp;
    sp.wgt = wgt + (b * h + hh0) * nc * Qp;
    sp.sgr = SEQ ? sgr + (b * h + hh0) * nc * Qp : nullptr;
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        sp.a2[k] = A[hh0 + k] * kLog2e;
        sp.bias[k] = dt_bias ? dt_bias[hh0 + k] : 0.f;
    }
    sp.softplus = softplus;
    sp.dt_min = dt_min;
    sp.dt_max = dt_max;
    sp.hrow = nc * Qp;
    sp.l = l;
    sp.Q = Q;
    sp.h = h;
    sp.Qp = Qp;

    f32x4 acc[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) acc[k] = zero4();
    float logdec = 0.f;

    // the first span's raw time steps are requested before the first blocks,
    // so that its per-row values are ready as soon as possible
    float dtv[K::NPASS], dav[K::NPASS];
    int rst[K::NPASS];
    sp_dt_load<IO, P, N, HPW, SEQ>(dtv, dav, rst, c, 0, sp, tid);
    SpBuf<IO, P, N, HPW> pa, pb;
    sp_prefetch(pa, c, 0, true, sp, tid);
    sp_prefetch(pb, c, 1, nsb > 1, sp, tid);

    // Two LDS buffers: block k + 1 is staged (buffer (k + 1) & 1, register
    // set pa / pb by parity) while block k is applied, one barrier per
    // block.  A span's weights are computed before its first block is
    // staged; the state decays by the new span's total after the previous
    // span's last block has been applied.
    {
        sp_span<IO, P, N, HPW, SEQ>(span, dtv, dav, rst, c, 0, sp, tid);
        float L = 0.f;
#pragma unroll
        for (int j = 0; j < SPAN; ++j) L += span.lam[hs][j];
        logdec = __builtin_bit_cast(float,
                                    __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, L)));
    }
    sp_stage(pa, lds0, span, 0, tid);
    sp_prefetch(pa, c, 2, 2 < nsb, sp, tid);
    lds_barrier();
    for (int k0 = 0; k0 < nsb; k0 += 2) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int k = k0 + half, nxt = k + 1;
            SpBuf<IO, P, N, HPW> &pn = half == 0 ? pb : pa;  // holds block nxt
            typename K::OP *const bk = half == 0 ? lds0 : lds1;
            typename K::OP *const bn = half == 0 ? lds1 : lds0;
            if (half == 0) wave_priority(progress_priority(k, nsb));
            const bool new_span = nxt < nsb && nxt % SPAN == 0;
            float L = 0.f;
            if (new_span) {
                sp_dt_load<IO, P, N, HPW, SEQ>(dtv, dav, rst, c, nxt, sp, tid);
                sp_span<IO, P, N, HPW, SEQ>(span, dtv, dav, rst, c, nxt, sp, tid);
#pragma unroll
                for (int j = 0; j < SPAN; ++j) L += span.lam[hs][j];
                L = __builtin_bit_cast(float,
                                       __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, L)));
            }
            if (nxt < nsb) sp_stage(pn, bn, span, nxt % SPAN, tid);
            sp_prefetch(pn, c, nxt + 2, nxt + 2 < nsb, sp, tid);
            if (k < nsb) sp_apply<IO, P, N, HPW>(acc, bk, hs, c0, lane);
            if (new_span) {
                const float decay = exp2_fast(L);
#pragma unroll
                for (int t = 0; t < TPW; ++t) acc[t] *= decay;
                logdec += L;
            }
            lds_barrier();
        }
    }
    // the last chunk's own state only feeds the final state
    if (c + 1 < nc || keep_last) {
        if constexpr (sizeof(IO) == 2) {
            // fp16 times a power of two per (batch, chunk, head): the head's
            // largest magnitude lands in [2^14, 2^15), so nothing overflows
            // and every element keeps fp16's 11 bits relative to that maximum
            float m = 0.f;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(acc[t][e]));
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
            if (lane == 0) wmax[wave] = m;
            lds_barrier();
#pragma unroll
            for (int k = 0; k < K::WPH; ++k) m = fmaxf(m, wmax[hs * K::WPH + k]);
            int ex = 0;
            frexpf(m, &ex);  // m = f 2^ex, f in [0.5, 1) (ex = 0 for m = 0)
            sp_store_t16<IO, P, N, HPW>(reinterpret_cast<f16 *>(St) + ((b * nc + c) * h + hh) * NP,
                                        acc, ldexpf(1.f, 15 - ex), c0, lane);
            if (c0 == 0 && lane == 0) Scl[(b * h + hh) * nc + c] = ldexpf(1.f, ex - 15);
        } else {
            sp_store_t<IO, P, N, HPW>(St + ((b * nc + c) * h + hh) * NP, acc, c0, lane);
        }
        if (c0 == 0 && lane == 0) Lam[(b * h + hh) * nc + c] = logdec;
    }
}

// ----------------------------------------------------------------------------
// 2. State scan: the serial pass over chunks,
//        H_0 = init (or 0),   H_{c+1} = 2^L_c H_c + S_c,
//    with S_c and L_c from k_chunk_state.  H_c is stored as chunk c's
//    boundary state in the read-out's matrix-core operand type (fp16 rounded
//    to nearest on the bf16 path, fp32 on the fp32 path), transposed
//    ([head_dim][state_dim]); the state after the last chunk is the final
//    state ([state_dim][head_dim]).  The recurrence itself runs in fp32.
//    One thread per 4 consecutive state elements of one (batch, head); the
//    chunk states are loaded 8 chunks ahead of their use.
__device__ __forceinline__ void store_state4(f16 *p, const f32x4 &v) {
    *reinterpret_cast<f16x4 *>(p) = f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
}
__device__ __forceinline__ void store_state4(float *p, const f32x4 &v) {
    *reinterpret_cast<f32x4 *>(p) = v;
}

// Block images for the chunk output (bf16 io): C and B of every 32-row block
// of every (batch, chunk, group) converted to fp16 and laid out exactly as
// the chunk output keeps them in LDS (swizzled, paired column order), so
// that it can copy a block straight from memory into LDS.  Image of block
// (b, c, gi, j): [C (T x N) | B (T x N)], fp16; rows past the chunk's or
// the sequence's end are zero.  One thread per 16-byte chunk of the image:
// in paired order, chunk 4m + g of a row holds columns 32m + 4g .. + 3 and
// 32m + 16 + 4g .. + 3, and the swizzle stores logical chunk k at k ^ f(r).
// Every thread of the state-scan grid converts image chunks in a grid-stride
// loop before its share of the scan, so the grid stays the scan's own size.
struct ImgArgs {
    const void *B, *C;  // io dtype [batch, seqlen, groups, N]
    f16 *img;
    int64_t l, Q, nc, nsb, pieces;
    int g;
};

template <typename IO, int N>
__device__ __forceinline__ void bc_image_piece(const ImgArgs &ia, int64_t q) {
    if constexpr (sizeof(IO) == 2) {
        constexpr int T = kT, CPR = N / 8;  // 16-byte chunks per row
        const int k = (int)(q % CPR);       // stored chunk
        q /= CPR;
        const int r = (int)(q % T);
        q /= T;
        const int which = (int)(q & 1);  // 0: C, 1: B
        q >>= 1;
        const int64_t blk = q;  // (b, c, gi, j) flattened
        const int j = (int)(blk % ia.nsb);
        const int64_t cgi = blk / ia.nsb;
        const int gi = (int)(cgi % ia.g);
        const int64_t bc = cgi / ia.g;
        const int64_t c = bc % ia.nc, b = bc / ia.nc;
        const int64_t row = (int64_t)j * T + r, t = c * ia.Q + row;
        const int kl = k ^ Swz<f16, N>::f(r);                 // logical chunk
        const int col = 32 * (kl >> 2) + 4 * (kl & 3);        // first of 4 + 4 columns
        u32x2 lo{0u, 0u}, hi{0u, 0u};
        if (row < ia.Q && t < ia.l) {
            const IO *src = static_cast<const IO *>(which ? ia.B : ia.C) +
                            ((b * ia.l + t) * ia.g + gi) * N + col;
            lo = *reinterpret_cast<const u32x2 *>(src);
            hi = *reinterpret_cast<const u32x2 *>(src + 16);
        }
        Row8v<IO> v;
        __builtin_memcpy(&v.e[0], &lo, 8);
        __builtin_memcpy(&v.e[4], &hi, 8);
        *reinterpret_cast<Row8v<f16> *>(ia.img + blk * (2 * T * N) + which * (T * N) + r * N +
                                        k * 8) = op_piece(v);
    }
}

// ROWS: the final state or the state after every chunk is written (the
// instance without them keeps fewer registers).
template <typename OP, typename IO, int N, bool ROWS>
__global__ __launch_bounds__(256) void k_state_scan(const float *__restrict__ St,
                                                    const float *__restrict__ Lam,
                                                    const float *__restrict__ Scl,
                                                    const float *__restrict__ init,
                                                    OP *__restrict__ Hb,
                                                    float *__restrict__ final_state, int64_t bh,
                                                    int h, int64_t nc, int n, int p,
                                                    ImgArgs ia, float *__restrict__ states) {
    constexpr int G8 = 8;
    __shared__ __attribute__((aligned(16))) float lds[4 * 256];
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = idx; q < ia.pieces; q += nthreads) bc_image_piece<IO, N>(ia, q);
    const int64_t np4 = (int64_t)n * p / 4;
    // threads past the last element stay for the barriers of the state
    // stores (computing on the last element, storing nothing)
    const bool live = idx < bh * np4;
    if (!ROWS) states = final_state = nullptr;
    if (!live && !ROWS) return;
    const int64_t ie = live ? idx : bh * np4 - 1;
    const ScanTile st(n, p);
    const int64_t tile = ie / st.TT;
    const int loc = (int)(ie % st.TT);
    const int64_t tpp = (int64_t)(n / st.R) * (p / st.Cc);  // tiles per state
    const int64_t pair = tile / tpp, tip = tile % tpp;
    const int row0 = (int)(tip % (n / st.R)) * st.R, col0 = (int)(tip / (n / st.R)) * st.Cc;
    const int64_t b = pair / h, hh = pair % h;
    // element e of this thread: head_dim column pc, state row n0 + e
    const int64_t n0 = row0 + (loc % (st.R / 4)) * 4, pc = col0 + loc / (st.R / 4);
    const int64_t e4 = (pc * n + n0) / 4;
    f32x4 H = zero4();
    if (init) {
        const float *src = init + pair * (int64_t)n * p + n0 * p + pc;
#pragma unroll
        for (int e = 0; e < 4; ++e) H[e] = src[e * p];
    }
    const int64_t cstride = (int64_t)h * np4;  // from one chunk to the next, in f32x4
    // chunk states: fp32, or (bf16 io) fp16 times the (batch, chunk, head) scale
    const f32x4 *S = reinterpret_cast<const f32x4 *>(St) + (b * nc * h + hh) * np4 + e4;
    const f16x4 *S16 = reinterpret_cast<const f16x4 *>(St) + (b * nc * h + hh) * np4 + e4;
    const float *Sc = Scl + pair * nc;
    OP *dst = Hb + ((b * nc * h + hh) * np4 + e4) * 4;
    const float *L = Lam + pair * nc;
    // chunks whose own state is needed: all but the last unless the final
    // state or the state after every chunk is asked for (the last chunk's
    // state is otherwise not even written)
    const int64_t ns = (final_state || states) ? nc : nc - 1;
    const int64_t klast = ns > 0 ? ns - 1 : 0;
    for (int64_t k0 = 0; k0 < nc; k0 += G8) {
        f32x4 Sk[G8];
        f16x4 Sh[G8];
        float Lk[G8], Ck[G8];
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int64_t k = k0 + u < klast ? k0 + u : klast;
            if constexpr (sizeof(IO) == 2) {
                Sh[u] = S16[k * cstride];
                Ck[u] = Sc[k];
            } else {
                Sk[u] = S[k * cstride];
            }
            Lk[u] = L[k];
        }
        if constexpr (sizeof(IO) == 2) {
#pragma unroll
            for (int u = 0; u < G8; ++u)
                Sk[u] = f32x4{(float)Sh[u][0], (float)Sh[u][1], (float)Sh[u][2], (float)Sh[u][3]} *
                        Ck[u];
        }
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            // the boundary state of chunk 0 is only stored for a given
            // initial state (the chunk output reads zeros otherwise)
            if (live && k0 + u < nc && (k0 + u > 0 || init))
                store_state4(dst + (k0 + u) * cstride * 4, H);
            if (k0 + u < ns) H = exp2_fast(Lk[u]) * H + Sk[u];
            // the state after chunk k0 + u, [b, nc, h, n, p]
            if (ROWS && states && k0 + u < nc)
                store_state_rows(lds, H, st, live,
                                 states + ((b * nc + k0 + u) * h + hh) * (int64_t)n * p, row0,
                                 col0, p);
        }
    }
    if (ROWS && final_state)
        store_state_rows(lds, H, st, live, final_state + pair * (int64_t)n * p, row0, col0, p);
}

// ----------------------------------------------------------------------------
// 3. Chunk output.  One workgroup per (batch, chunk, HPW consecutive heads of
//    one group); WPH = max(1, head_dim / 32) waves per head, each owning 32
//    (or head_dim, if smaller) head_dim columns.  C and B of a block are
//    staged once for all the workgroup's heads (they share the group), x per
//    head.  A wave keeps its columns of the running state H (all state_dim
//    rows) in MFMA accumulators across the chunk's blocks.  Per block:
//      G^T = B C^T on the 3 causal 16 x 16 tiles, and
//      P_ij = G_ij 2^(lcs_i - lcs_j) d_j (j <= i), in registers;
//      y^T = 2^lcs_i (H^T C^T) + x^T (P + D I)^T (the skip term on the
//            scores' diagonal), stored straight from the
//            accumulators (4 consecutive columns per lane);
//      H <- 2^lcs_last H + B^T (w x)  (except after the last block).
//    The scores and the state read-out take the same C fragments (one LDS
//    read for both).  The decay factor of P is taken as a_i b_j with
//    a_i = 2^(lcs_i - lcs_15) and b_j = 2^(lcs_15 - lcs_j) d_j, both per
//    row, when the block's total log2 decay is above -kSplitLimit (every
//    factor then stays inside fp32's normal range); otherwise as one
//    exponential per element.
constexpr float kSplitLimit = 60.f;

template <typename IO, int P, int N, int HPW, bool COPY = (sizeof(IO) == 2)> struct Co {
    typedef typename Op<IO>::type OP;
    typedef Mfma<OP> M;
    static constexpr int T = kT;
    static constexpr int WPH = P >= 64 ? P / 32 : 1;  // waves per head
    static constexpr int PW = P / WPH;                // head_dim columns per wave
    static constexpr int CPW = PW / 16;               // column tiles per wave
    static constexpr int W = HPW * WPH, NT = 64 * W;  // waves, threads
    static constexpr int RT = N / 16;                 // state row tiles
    static constexpr int NB = N / 32;                 // 32-blocks of the state index
    static constexpr int KS = T / M::K;               // MFMA steps per 32-block
    // COPY (bf16 io only): blocks are copied into LDS by the buffer unit (C
    // and B from their fp16 block images, x as raw bf16 in rows of head_dim
    // elements); otherwise staged through registers, x rows padded
    static constexpr bool DMA = COPY && sizeof(IO) == 2;
    static constexpr int LDX = DMA ? P : P + 16;      // [row][p]: x
    static constexpr int XS = T * LDX;                // one head's staged x
    static constexpr int BUF = 2 * T * N + HPW * XS;  // [C | B | x of each head]
    // staging pieces (8 elements) per thread (fp32 io)
    static constexpr int NPC = T * N / 8, NPX = HPW * T * P / 8;
    static constexpr int KC = (NPC + NT - 1) / NT, KX = (NPX + NT - 1) / NT;
    // 16-byte copies per block (bf16 io): C and B image, x of all heads
    static constexpr int CBQ = T * N / 4, XQ = HPW * T * P / 8;
    static constexpr int ND = DMA ? (CBQ + XQ) / NT : 0;  // copy instructions per thread
    static_assert(!DMA || (CBQ % NT == 0 && XQ % NT == 0), "whole copy rounds per wave");
    // buffer stores of y per thread and block
    static constexpr int NS = CPW % 2 == 0 ? CPW * (DMA ? 1 : 2) : 2 * CPW;
};

// Raw bf16 x in LDS (bf16 io): row r of a head holds head_dim elements in
// 16-byte chunks, chunk k at position k ^ xsw(r).  With 8-byte pieces read
// by the transposing loads, this leaves at most two lanes per bank.
template <int P> __device__ __forceinline__ int xsw(int r) {
    return ((((r >> 1) & 3) << 2)) & (P / 8 - 1);
}
template <int P> __device__ __forceinline__ int xsw_at(int r, int col) {
    return r * P + (((col >> 3) ^ xsw<P>(r)) << 3) + (col & 7);
}


// Per-row factors of one head's staged block (LDS), T floats each.
// Values read per output row i are kept in pairs (i, i + 16), so that a lane
// reads the two rows it owns with one 8-byte access.
struct alignas(16) CoRows {
    float lcs[kT];   // cumulative log2 decay inside the block
    float d[kT];     // time step
    float a2[kT];    // 2^(lcs_i - lcs_15), pairs (i, i + 16) at 2 (i % 16)
    float l2[kT];    // lcs_i in the same pairs
    float bw[kT];    // 2^(lcs_15 - lcs_j) d_j
    float w[kT];     // 2^(lcs_31 - lcs_j) d_j: weight in the state at the block's end
    int seg[kT];     // packed sequences: the last row <= i of the block that starts
                     // from a zero state, or -1
};
__device__ __forceinline__ int row_pair(int r) { return 2 * (r & 15) + (r >> 4); }

// Row factors of one block, loaded by thread tid for head tid / kT, row
// tid % kT (threads past HPW * kT load and discard).
struct CoRowV {
    float ls, ds, ws, l15;
    int sg;  // packed sequences: the row's last reset in its block, or -1
};

// Register prefetch of one block for the whole workgroup (fp32 io).  Loads
// go through buffer resources that end at the chunk's last valid row (zeros
// beyond).
template <typename IO, int P, int N, int HPW> struct CoBuf {
    typedef Co<IO, P, N, HPW, false> K;
    typedef typename K::OP OP;
    Row8v<IO> cv[K::KC], bv[K::KC];
    Row8v<IO> xv[K::KX];
    CoRowV r;
};

// Per-workgroup addressing.
template <typename IO> struct CoPtrs {
    typedef typename Op<IO>::type OP;
    const IO *x;        // row 0 of the chunk, first head of the workgroup
    const IO *B, *C;    // row 0 of the chunk, the group
    IO *y;
    Rsrc rl, rd, rw;    // lcs, d, weights: the workgroup's heads, this chunk
    int64_t xs, bs;     // row strides (elements) of x / y and of B / C
    uint32_t hstride;   // bytes from one head's row arrays to the next
    int rows;           // valid rows of the chunk
    Rsrc rimg;          // block images of this (batch, chunk, group) (bf16 io)
    Rsrc rsg;           // packed sequences: the rows' last resets (as rl)
    int64_t t0;         // the chunk's first token
};

// Vector memory loads co_rows_prefetch issues per thread.
template <bool SEQ> constexpr int kRowLoads = SEQ ? 5 : 4;

template <int HPW, bool SEQ, typename IO>
__device__ __forceinline__ void co_rows_prefetch(CoRowV &f, int s, const CoPtrs<IO> &cp, int tid) {
    constexpr int T = kT;
    const int hs = tid < HPW * T ? tid / T : 0, row = tid % T;
    const uint32_t soff = (uint32_t)(s * T) * 4u;
    const uint32_t ro = (uint32_t)hs * cp.hstride + (uint32_t)row * 4u;
    f.ls = buf_f32(cp.rl, ro, soff);
    f.ds = buf_f32(cp.rd, ro, soff);
    f.ws = buf_f32(cp.rw, ro, soff);
    f.l15 = buf_f32(cp.rl, (uint32_t)hs * cp.hstride + 15u * 4u, soff);
    if constexpr (SEQ) f.sg = __builtin_bit_cast(int, buf_f32(cp.rsg, ro, soff));
}

template <int HPW, bool SEQ>
__device__ __forceinline__ void co_rows_stage(const CoRowV &f, CoRows *rows, int tid) {
    constexpr int T = kT;
    if (tid < HPW * T) {
        CoRows &rw = rows[tid / T];
        const int r = tid % T;
        if constexpr (SEQ) rw.seg[r] = f.sg;
        rw.lcs[r] = f.ls;
        rw.d[r] = f.ds;
        rw.a2[row_pair(r)] = exp2_fast(f.ls - f.l15);
        rw.l2[row_pair(r)] = f.ls;
        rw.bw[r] = exp2_fast(f.l15 - f.ls) * f.ds;
        rw.w[r] = f.ws;
    }
}

// bf16 io: block s copied into LDS buffer buf by the buffer unit, 16 bytes
// per lane and instruction, each wave filling 1 KB of consecutive LDS per
// instruction: C and B from the block image (already in LDS order), x as
// raw bf16 with each lane fetching the 16-byte chunk its LDS slot holds.
// Rows past the chunk's end read as zeros.  Issues exactly K::ND copies per
// thread.
template <typename IO, int P, int N, int HPW>
__device__ __forceinline__ void co_dma(typename Op<IO>::type *buf, int s, const CoPtrs<IO> &cp,
                                       int wave, int lane) {
    typedef Co<IO, P, N, HPW, true> K;
    constexpr int T = kT, CH = P / 8;
#pragma unroll
    for (int q0 = 0; q0 < K::CBQ; q0 += K::NT) {
        const int q = q0 + wave * 64;
        lds_copy16(cp.rimg, (lds_void *)(buf + q * 8), (uint32_t)((s * K::CBQ + q + lane) * 16));
    }
    const int r0 = s * T;
    int valid = cp.rows - r0;
    valid = valid < 0 ? 0 : (valid > T ? T : valid);
    const Rsrc rx = make_rsrc(cp.x + (valid > 0 ? r0 : 0) * cp.xs,
                              (int64_t)valid * cp.xs * (int)sizeof(IO));
    typename Op<IO>::type *Xs = buf + 2 * T * N;
#pragma unroll
    for (int q0 = 0; q0 < K::XQ; q0 += K::NT) {
        const int qw = q0 + wave * 64, q = qw + lane;
        const int hs = q / (T * CH), rem = q % (T * CH), r = rem / CH, k = rem % CH;
        const uint32_t off =
            (uint32_t)(r * cp.xs + hs * P + ((k ^ xsw<P>(r)) << 3)) * (uint32_t)sizeof(IO);
        lds_copy16(rx, (lds_void *)(Xs + qw * 8), off);
    }
}

template <bool SEQ, typename IO, int P, int N, int HPW>
__device__ __forceinline__ void co_prefetch(CoBuf<IO, P, N, HPW> &f, int s, const CoPtrs<IO> &cp,
                                            int tid) {
    typedef Co<IO, P, N, HPW, false> K;
    typedef typename K::OP OP;
    constexpr int T = kT;
    const int r0 = s * T;
    int valid = cp.rows - r0;
    valid = valid < 0 ? 0 : (valid > T ? T : valid);
    const int rr0 = valid > 0 ? r0 : 0;
    const Rsrc rb = make_rsrc(cp.B + rr0 * cp.bs, (int64_t)valid * cp.bs * (int)sizeof(IO));
    const Rsrc rc = make_rsrc(cp.C + rr0 * cp.bs, (int64_t)valid * cp.bs * (int)sizeof(IO));
    const Rsrc rx = make_rsrc(cp.x + rr0 * cp.xs, (int64_t)valid * cp.xs * (int)sizeof(IO));
#pragma unroll
    for (int k = 0; k < K::KC; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPC % K::NT == 0 || q < K::NPC) {
            const int j = q / (N / 8), cc = q % (N / 8);
            const uint32_t off = (uint32_t)(j * cp.bs + cc * 8) * (uint32_t)sizeof(IO);
            f.cv[k] = buf_row8<IO>(rc, off);
            f.bv[k] = buf_row8<IO>(rb, off);
        }
    }
#pragma unroll
    for (int k = 0; k < K::KX; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPX % K::NT == 0 || q < K::NPX) {
            const int hs = q / (T * P / 8), qq = q % (T * P / 8);
            const int j = qq / (P / 8), cc = qq % (P / 8);
            f.xv[k] = buf_row8<IO>(rx, (uint32_t)(j * cp.xs + hs * P + cc * 8) *
                                           (uint32_t)sizeof(IO));
        }
    }
    co_rows_prefetch<HPW, SEQ>(f.r, s, cp, tid);
}

template <bool SEQ, typename IO, int P, int N, int HPW>
__device__ __forceinline__ void co_stage(const CoBuf<IO, P, N, HPW> &f,
                                         typename Op<IO>::type *buf, CoRows *rows, int tid) {
    typedef Co<IO, P, N, HPW, false> K;
    typedef typename K::OP OP;
    constexpr int T = kT;
    OP *Cs = buf, *Bs = buf + T * N, *Xs = buf + 2 * T * N;
#pragma unroll
    for (int k = 0; k < K::KC; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPC % K::NT == 0 || q < K::NPC) {
            const int r = q / (N / 8), c0 = (q % (N / 8)) * 8;
            if constexpr (sizeof(OP) == 2) {
                swzp_store8<N>(Cs, r, c0, op_piece(f.cv[k]));
                swzp_store8<N>(Bs, r, c0, op_piece(f.bv[k]));
            } else {
                swz_store8<OP, N>(Cs, r, c0, op_piece(f.cv[k]));
                swz_store8<OP, N>(Bs, r, c0, op_piece(f.bv[k]));
            }
        }
    }
#pragma unroll
    for (int k = 0; k < K::KX; ++k) {
        const int q = tid + k * K::NT;
        if (K::NPX % K::NT == 0 || q < K::NPX) {
            const int hs = q / (T * P / 8), qq = q % (T * P / 8);
            st_row8(Xs + hs * K::XS + (qq / (P / 8)) * K::LDX + (qq % (P / 8)) * 8,
                    op_piece(f.xv[k]));
        }
    }
    co_rows_stage<HPW, SEQ>(f.r, rows, tid);
}

// Decay-weighted x, w_j x_j, as the k-major B operand of the state carry:
// the x fragment scaled row by row (rows 4g + r and 16 + 4g + r of lane
// group g; fp32: row 16 (q >> 2) + 4g + (q & 3)).
__device__ __forceinline__ f16x8 xw_frag(const f16x8 &xf, int q, int lane, const float *w) {
    const int g = lane >> 4;
    const f32x4 wa = *reinterpret_cast<const f32x4 *>(w + 4 * g);
    const f32x4 wb = *reinterpret_cast<const f32x4 *>(w + 16 + 4 * g);
    const f16x2 o0 = pk2((float)xf[0] * wa[0], (float)xf[1] * wa[1]);
    const f16x2 o1 = pk2((float)xf[2] * wa[2], (float)xf[3] * wa[3]);
    const f16x2 o2 = pk2((float)xf[4] * wb[0], (float)xf[5] * wb[1]);
    const f16x2 o3 = pk2((float)xf[6] * wb[2], (float)xf[7] * wb[3]);
    return f16x8{o0[0], o0[1], o1[0], o1[1], o2[0], o2[1], o3[0], o3[1]};
}
__device__ __forceinline__ float xw_frag(float xf, int q, int lane, const float *w) {
    return xf * w[16 * (q >> 2) + 4 * (lane >> 4) + (q & 3)];
}

// head_dim column of row rho (0..15) of the wave's column tile u.  Tiles are
// taken in pairs that interleave in groups of 4 columns (tile 2v holds
// columns 32v + 8m + e, tile 2v + 1 holds 32v + 8m + 4 + e, m, e < 4), so that
// a lane's output rows of the two tiles are 8 consecutive columns.
template <int CPW> __device__ __forceinline__ int co_col(int u, int rho) {
    if constexpr (CPW % 2 == 0)
        return 32 * (u >> 1) + 8 * (rho >> 2) + 4 * (u & 1) + (rho & 3);
    else
        return 16 * u + rho;
}

// k-major x fragment of column tile u (rows = block rows, columns co_col).
template <int CPW>
__device__ __forceinline__ f16x8 xs_frag(const f16 *Xs, int ldx, int q, int c0, int u, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int col = c0 + co_col<CPW>(u, 4 * (j & 3));
    const f16 *pa = Xs + (4 * g + (j >> 2)) * ldx + col;
    const f16 *pb = Xs + (16 + 4 * g + (j >> 2)) * ldx + col;
    const f16x4 a = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pa));
    const f16x4 b = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pb));
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <int CPW>
__device__ __forceinline__ float xs_frag(const float *Xs, int ldx, int q, int c0, int u, int lane) {
    return Xs[(16 * (q >> 2) + 4 * (lane >> 4) + (q & 3)) * ldx + c0 + co_col<CPW>(u, lane & 15)];
}

// The same fragment from raw bf16 x in the swizzled rows of the copied
// layout, converted to fp16 operands (exact bf16 -> fp32, then rounded
// toward zero, as the register-staged path does).
template <int CPW, int P>
__device__ __forceinline__ f16x8 xs_frag_raw(const f16 *Xs, int c0, int u, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int col = c0 + co_col<CPW>(u, 4 * (j & 3));
    const int ra = 4 * g + (j >> 2), rb = 16 + ra;
    const u32x2 a = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(Xs + xsw_at<P>(ra, col))));
    const u32x2 b = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(Xs + xsw_at<P>(rb, col))));
    const u32x4 w{a[0], a[1], b[0], b[1]};
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16x2 pk = pk2(__builtin_bit_cast(float, w[i] << 16),
                             __builtin_bit_cast(float, w[i] & 0xffff0000u));
        o[2 * i] = pk[0];
        o[2 * i + 1] = pk[1];
    }
    return o;
}

// One block of the chunk output for one wave: head slot hs, columns
// c0 .. c0 + PW - 1 of that head.  accH: the wave's CPW x RT state tiles
// (inlined: stays in registers).
template <typename IO, int P, int N, int HPW, bool COPY, bool SEQ>
__device__ __forceinline__ void co_compute(f32x4 *accH, const typename Op<IO>::type *buf,
                                           const CoRows &rf, bool carry, float Dh,
                                           const CoPtrs<IO> &cp, int r0, int hs, int c0,
                                           int lane) {
    typedef Co<IO, P, N, HPW, COPY> K;
    typedef typename K::OP OP;
    typedef typename K::M M;
    constexpr int T = kT, KS = K::KS, NB = K::NB, LDX = K::LDX, CPW = K::CPW, RT = K::RT;
    const int lg = lane >> 4, li = lane & 15;
    const OP *Cs = buf;
    const OP *Bs = buf + T * N;
    const OP *Xs = buf + 2 * T * N + hs * K::XS;

    // ---- G^T tiles and the state read-out, sharing the C fragments.
    //      gt[k]: tiles (it, jt) = (0,0), (1,0), (1,1); element r of lane l:
    //      j = 16 jt + 4 lg + r, i = 16 it + li.  yh[it][u]: H^T C^T for
    //      rows 16 it.. and columns c0 + 16 u..
    f32x4 gt[3], yh[2][CPW];
#pragma unroll
    for (int k = 0; k < 3; ++k) gt[k] = zero4();
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int u = 0; u < CPW; ++u) yh[it][u] = zero4();
#pragma unroll
    for (int m = 0; m < NB; ++m) {
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            typename M::frag c0f, c1f, b0f, b1f;
            if constexpr (sizeof(OP) == 2) {
                c0f = swzp_rows_kconv<N>(Cs, 0, 32 * m, lane);
                c1f = swzp_rows_kconv<N>(Cs, 16, 32 * m, lane);
                b0f = swzp_rows_kconv<N>(Bs, 0, 32 * m, lane);
                b1f = swzp_rows_kconv<N>(Bs, 16, 32 * m, lane);
            } else {
                c0f = swz_rows_kconv<OP, N>(Cs, 0, 32 * m, q, lane);
                c1f = swz_rows_kconv<OP, N>(Cs, 16, 32 * m, q, lane);
                b0f = swz_rows_kconv<OP, N>(Bs, 0, 32 * m, q, lane);
                b1f = swz_rows_kconv<OP, N>(Bs, 16, 32 * m, q, lane);
            }
            gt[0] = M::mma(b0f, c0f, gt[0]);
            gt[1] = M::mma(b0f, c1f, gt[1]);
            gt[2] = M::mma(b1f, c1f, gt[2]);
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const auto hf = frag_from_acc<OP>(accH[u * RT + 2 * m], accH[u * RT + 2 * m + 1], q);
                yh[0][u] = M::mma(hf, c0f, yh[0][u]);
                yh[1][u] = M::mma(hf, c1f, yh[1][u]);
            }
        }
    }

    // ---- masked, decayed scores pv[it][jt] (registers)
    const float lam = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, rf.lcs[T - 1])));
    f32x4 pv[2][2];
    float colscale[2];
    pv[0][1] = zero4();
    if (lam > -kSplitLimit) {
        const float s15 = exp2_fast(rf.lcs[15]);
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&rf.bw[4 * lg]);
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&rf.bw[16 + 4 * lg]);
        const f32x2 ap = *reinterpret_cast<const f32x2 *>(&rf.a2[2 * li]);
        const float a0 = ap[0], a1 = ap[1];
        colscale[0] = a0 * s15;
        colscale[1] = a1 * s15;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j0 = 4 * lg + r;
            pv[0][0][r] = (j0 <= li) ? gt[0][r] * (a0 * b0[r]) : 0.f;
            pv[1][0][r] = gt[1][r] * (a1 * b0[r]);
            pv[1][1][r] = (j0 <= li) ? gt[2][r] * (a1 * b1[r]) : 0.f;
        }
    } else {
        const f32x2 lp = *reinterpret_cast<const f32x2 *>(&rf.l2[2 * li]);
        const float l0 = lp[0], l1 = lp[1];
        colscale[0] = exp2_fast(l0);
        colscale[1] = exp2_fast(l1);
        if constexpr (K::DMA) {
            // whole 16-byte reads: the compiler can then tell them from the
            // block copies in flight and does not wait for those
            const f32x4 lj0 = *reinterpret_cast<const f32x4 *>(&rf.lcs[4 * lg]);
            const f32x4 lj1 = *reinterpret_cast<const f32x4 *>(&rf.lcs[16 + 4 * lg]);
            const f32x4 dj0 = *reinterpret_cast<const f32x4 *>(&rf.d[4 * lg]);
            const f32x4 dj1 = *reinterpret_cast<const f32x4 *>(&rf.d[16 + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j0 = 4 * lg + r;
                pv[0][0][r] = (j0 <= li) ? gt[0][r] * exp2_fast(l0 - lj0[r]) * dj0[r] : 0.f;
                pv[1][0][r] = gt[1][r] * exp2_fast(l1 - lj0[r]) * dj0[r];
                pv[1][1][r] = (j0 <= li) ? gt[2][r] * exp2_fast(l1 - lj1[r]) * dj1[r] : 0.f;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j0 = 4 * lg + r;
                pv[0][0][r] = (j0 <= li) ? gt[0][r] * exp2_fast(l0 - rf.lcs[j0]) * rf.d[j0] : 0.f;
                pv[1][0][r] = gt[1][r] * exp2_fast(l1 - rf.lcs[j0]) * rf.d[j0];
                pv[1][1][r] =
                    (j0 <= li) ? gt[2][r] * exp2_fast(l1 - rf.lcs[16 + j0]) * rf.d[16 + j0] : 0.f;
            }
        }
    }
    if constexpr (SEQ) {
        // packed sequences: scores only between rows of one document, and
        // the state entering the block only for rows before its first reset
        const int sA = rf.seg[li], sB = rf.seg[16 + li];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j0 = 4 * lg + r;
            if (j0 < sA) pv[0][0][r] = 0.f;
            if (j0 < sB) pv[1][0][r] = 0.f;
            if (16 + j0 < sB) pv[1][1][r] = 0.f;
        }
        if (sA >= 0) colscale[0] = 0.f;
        if (sB >= 0) colscale[1] = 0.f;
    }
    // the skip term rides on the diagonal: (P + D I) x = P x + D x
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float dg = 4 * lg + r == li ? Dh : 0.f;
        pv[0][0][r] += dg;
        pv[1][1][r] += dg;
    }

    // ---- y^T = colscale (H^T C^T) + x^T (P + D I)^T, straight to y:
    //      element r of lane l is (p = c0 + co_col(u, 4 lg + r), i = 16 it + li)
    int valid = cp.rows - r0;
    valid = valid < 0 ? 0 : (valid > T ? T : valid);
    const Rsrc ry = make_rsrc(cp.y + (valid > 0 ? r0 : 0) * cp.xs,
                              (int64_t)valid * cp.xs * (int)sizeof(IO));
    typename Mfma<OP>::frag xf[CPW][KS];
#pragma unroll
    for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            if constexpr (K::DMA)
                xf[u][q] = xs_frag_raw<CPW, P>(Xs, c0, u, lane);
            else
                xf[u][q] = xs_frag<CPW>(Xs, LDX, q, c0, u, lane);
        }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int i = it * 16 + li;
        f32x4 yv[CPW];
        (void)LDX;
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            f32x4 yp = zero4();
#pragma unroll
            for (int q = 0; q < KS; ++q)
                yp = M::mma(xf[u][q], frag_from_acc<OP>(pv[it][0], pv[it][1], q), yp);
            yv[u] = colscale[it] * yh[it][u] + yp;
        }
        if constexpr (CPW % 2 == 0) {
            // tiles 2v, 2v + 1: 8 consecutive columns c0 + 32 v + 8 lg ..
#pragma unroll
            for (int v = 0; v < CPW / 2; ++v) {
                const f32x4 lo = yv[2 * v], hi = yv[2 * v + 1];
                const uint32_t off = (uint32_t)(i * cp.xs + hs * P + c0 + 32 * v + 8 * lg) *
                                     (uint32_t)sizeof(IO);
                if constexpr (sizeof(IO) == 2) {
                    const bf16x4 a{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3]};
                    const bf16x4 bq{(bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
                    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, bq);
                    buf_store16(ry, off, u32x4{ua[0], ua[1], ub[0], ub[1]});
                } else {
                    buf_store16(ry, off, __builtin_bit_cast(u32x4, lo));
                    buf_store16(ry, off + 16u, __builtin_bit_cast(u32x4, hi));
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const uint32_t off = (uint32_t)(i * cp.xs + hs * P + c0 + co_col<CPW>(u, 4 * lg)) *
                                     (uint32_t)sizeof(IO);
                if constexpr (sizeof(IO) == 2) {
                    const bf16x4 o{(bf16)yv[u][0], (bf16)yv[u][1], (bf16)yv[u][2], (bf16)yv[u][3]};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), ry, off, 0,
                                                          0);
                } else {
                    buf_store16(ry, off, __builtin_bit_cast(u32x4, yv[u]));
                }
            }
        }
    }

    // ---- carry the state to the next block of the chunk
    if (carry) {
        // packed sequences: nothing carried across a reset in the block
        const float decay = (SEQ && rf.seg[T - 1] >= 0) ? 0.f : exp2_fast(lam);
        typename Mfma<OP>::frag xw[CPW][KS];
#pragma unroll
        for (int u = 0; u < CPW; ++u)
#pragma unroll
            for (int q = 0; q < KS; ++q) xw[u][q] = xw_frag(xf[u][q], q, lane, rf.w);
#pragma unroll
        for (int k = 0; k < CPW * RT; ++k) accH[k] *= decay;
#pragma unroll
        for (int tr = 0; tr < RT; ++tr)
#pragma unroll
            for (int q = 0; q < KS; ++q) {
                typename M::frag bt;
                if constexpr (sizeof(OP) == 2)
                    bt = swzp_kmajor<N>(Bs, 0, tr * 16, lane);
                else
                    bt = swz_kmajor<OP, N>(Bs, 0, q, tr * 16, lane);
#pragma unroll
                for (int u = 0; u < CPW; ++u)
                    accH[u * RT + tr] = M::mma(bt, xw[u][q], accH[u * RT + tr]);
            }
    }
}

// copying path: three workgroups per compute unit, also with packed
// sequences (whose row masks then spill a few bytes at state_dim 128, which
// still beats two workgroups per CU: 44.6 -> 39.0 us at the 130m shape)
template <typename IO, int P, int N, int HPW, bool COPY, bool SEQ>
__global__ __launch_bounds__((Co<IO, P, N, HPW, COPY>::NT),
                             (Co<IO, P, N, HPW, COPY>::DMA ? 3 : 1)) void k_chunk_out(
    const IO *__restrict__ x, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ lcs, const float *__restrict__ dtp,
    const float *__restrict__ wgt, const typename Op<IO>::type *__restrict__ Hb,
    IO *__restrict__ y, int64_t l, int h, int g, int64_t Q, int64_t nc, int64_t Qp,
    const f16 *__restrict__ img, int64_t nsb, int has_init, const int *__restrict__ sgr) {
    typedef Co<IO, P, N, HPW, COPY> K;
    typedef typename K::OP OP;
    constexpr int T = kT, BUF = K::BUF, CPW = K::CPW, RT = K::RT, WPH = K::WPH;
    // two block buffers as separate objects, so that the compiler can tell
    // a copy into one from reads of the other
    __shared__ __attribute__((aligned(16))) OP lds0[BUF];
    __shared__ __attribute__((aligned(16))) OP lds1[BUF];
    __shared__ CoRows rows0[HPW];
    __shared__ CoRows rows1[HPW];

    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int lg = lane >> 4, li = lane & 15;
    int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int hq = (int)(item % (h / HPW)); item /= (h / HPW);
    const int64_t c = item % nc;
    const int64_t b = item / nc;
    const int hh0 = hq * HPW;                // first head of the workgroup
    const int gi = hh0 / (h / g);
    const int hs = wave / WPH;               // this wave's head slot
    const int hh = hh0 + hs;
    const int c0 = (wave % WPH) * K::PW;     // this wave's first column
    const int64_t NP = (int64_t)N * P;
    const int64_t t0 = c * Q;
    CoPtrs<IO> cp;
    cp.xs = (int64_t)h * P;
    cp.bs = (int64_t)g * N;
    cp.x = x + ((b * l + t0) * h + hh0) * P;
    cp.y = y + ((b * l + t0) * h + hh0) * P;
    cp.B = Bm + ((b * l + t0) * g + gi) * N;
    cp.C = Cm + ((b * l + t0) * g + gi) * N;
    const int64_t rbase = ((b * h + hh0) * nc + c) * Qp;
    const int64_t rspan = ((int64_t)(HPW - 1) * nc * Qp + Qp) * 4;
    cp.rl = make_rsrc(lcs + rbase, rspan);
    cp.rd = make_rsrc(dtp + rbase, rspan);
    cp.rw = make_rsrc(wgt + rbase, rspan);
    cp.hstride = (uint32_t)(nc * Qp * 4);
    cp.rows = (int)((Q < l - t0) ? Q : (l - t0));
    cp.t0 = t0;
    if constexpr (SEQ) cp.rsg = make_rsrc(sgr + rbase, rspan);
    if constexpr (K::DMA)
        cp.rimg = make_rsrc(img + ((b * nc + c) * g + gi) * nsb * (2 * T * N),
                            nsb * (int64_t)(4 * T * N));
    const int nblk = (cp.rows + T - 1) / T;
    const float Dh = D ? D[hh] : 0.f;

    OP *const buf0 = lds0;
    OP *const buf1 = lds1;

    // ---- the wave's state columns entering the chunk: the boundary state,
    //      stored transposed ([head_dim][state_dim]) in the operand type, so
    //      a lane's 4 accumulator values (consecutive state rows) are one
    //      load.  Loaded after the first block is requested, so that staging
    //      block 0 does not wait for them.
    typedef typename std::conditional<sizeof(OP) == 2, f16x4, f32x4>::type HRaw;
    HRaw hraw[CPW * RT];
    auto load_boundary = [&]() {
        // chunk 0 from a zero initial state: nothing stored, loads read zeros
        const int64_t hbytes = (c > 0 || has_init) ? NP * (int64_t)sizeof(OP) : 0;
        const Rsrc rh = make_rsrc(Hb + ((b * nc + c) * h + hh) * NP, hbytes);
#pragma unroll
        for (int u = 0; u < CPW; ++u)
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) {
                const uint32_t off = (uint32_t)((c0 + co_col<CPW>(u, li)) * N + tr * 16 + 4 * lg) *
                                     (uint32_t)sizeof(OP);
                if constexpr (sizeof(OP) == 2)
                    hraw[u * RT + tr] = __builtin_bit_cast(
                        f16x4, __builtin_amdgcn_raw_buffer_load_b64(rh, off, 0, 0));
                else
                    hraw[u * RT + tr] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, off, 0, 0));
            }
    };
    f32x4 accH[CPW * RT];

    if constexpr (K::DMA) {
        // Block k is copied into LDS buffer k & 1 (its row factors into
        // registers ra / rb) one block ahead: the copy of block k + 1 is in
        // flight while block k is computed.  Before each barrier a wave waits
        // for its own copies of the next block; only the y stores of the
        // block just computed may still be in flight then.  Blocks go in
        // pairs with every copy and store issued unconditionally (past the
        // chunk's end the copies read zeros and a block computed on them
        // stores nothing), so every wave issues the same operations and the
        // counts waited for are exact.
        CoRowV ra, rb;
        co_dma<IO, P, N, HPW>(buf0, 0, cp, wave, lane);
        co_rows_prefetch<HPW, SEQ>(ra, 0, cp, tid);
        issue_fence();
        load_boundary();
        issue_fence();
        co_dma<IO, P, N, HPW>(buf1, 1, cp, wave, lane);
        co_rows_prefetch<HPW, SEQ>(rb, 1, cp, tid);
        issue_fence();
        vm_wait<K::ND + kRowLoads<SEQ>>();  // block 0 and the boundary state have landed
        co_rows_stage<HPW, SEQ>(ra, rows0, tid);
        lds_barrier();
#pragma unroll
        for (int k = 0; k < CPW * RT; ++k)
            accH[k] = f32x4{(float)hraw[k][0], (float)hraw[k][1], (float)hraw[k][2], (float)hraw[k][3]};
        for (int s = 0; s < nblk; s += 2) {
            wave_priority(progress_priority(s, nblk));
            co_compute<IO, P, N, HPW, COPY, SEQ>(accH, buf0, rows0[hs], s + 1 < nblk, Dh, cp, s * T, hs,
                                      c0, lane);
            vm_wait<K::NS>();  // block s + 1
            co_rows_stage<HPW, SEQ>(rb, rows1, tid);
            lds_barrier();
            co_dma<IO, P, N, HPW>(buf0, s + 2, cp, wave, lane);
            co_rows_prefetch<HPW, SEQ>(ra, s + 2, cp, tid);
            issue_fence();
            co_compute<IO, P, N, HPW, COPY, SEQ>(accH, buf1, rows1[hs], s + 2 < nblk, Dh, cp, (s + 1) * T,
                                      hs, c0, lane);
            vm_wait<K::NS>();  // block s + 2
            co_rows_stage<HPW, SEQ>(ra, rows0, tid);
            lds_barrier();
            co_dma<IO, P, N, HPW>(buf1, s + 3, cp, wave, lane);
            co_rows_prefetch<HPW, SEQ>(rb, s + 3, cp, tid);
            issue_fence();
        }
        // no copy may still be writing this workgroup's LDS when it exits
        vm_wait<0>();
    } else {
        // Block k is fetched into registers pa (k even) or pb (k odd) two
        // blocks ahead and staged into LDS buffer k & 1 while block k - 1 is
        // computed.  Blocks go in pairs, every load and store issued
        // unconditionally (past the chunk's end: empty resources; a block
        // past the end is computed on zeros and stores nothing), so the loop
        // has one path and the memory counters never need a full drain.
        CoBuf<IO, P, N, HPW> pa, pb;
        co_prefetch<SEQ>(pa, 0, cp, tid);
        co_prefetch<SEQ>(pb, 1, cp, tid);
        load_boundary();
        co_stage<SEQ>(pa, buf0, rows0, tid);
        co_prefetch<SEQ>(pa, 2, cp, tid);
        lds_barrier();
#pragma unroll
        for (int k = 0; k < CPW * RT; ++k)
            accH[k] = f32x4{(float)hraw[k][0], (float)hraw[k][1], (float)hraw[k][2], (float)hraw[k][3]};
        for (int s = 0; s < nblk; s += 2) {
            co_stage<SEQ>(pb, buf1, rows1, tid);  // block s + 1
            co_prefetch<SEQ>(pb, s + 3, cp, tid);
            co_compute<IO, P, N, HPW, COPY, SEQ>(accH, buf0, rows0[hs], s + 1 < nblk, Dh, cp, s * T, hs,
                                      c0, lane);
            lds_barrier();
            co_stage<SEQ>(pa, buf0, rows0, tid);  // block s + 2
            co_prefetch<SEQ>(pa, s + 4, cp, tid);
            co_compute<IO, P, N, HPW, COPY, SEQ>(accH, buf1, rows1[hs], s + 2 < nblk, Dh, cp, (s + 1) * T,
                                      hs, c0, lane);
            lds_barrier();
        }
    }
}

// ----------------------------------------------------------------------------
template <typename IO, int P, int N>
hipError_t launch_scan(const ScanPlan &pl, const ScanArgs &a, hipStream_t s) {
    typedef typename Op<IO>::type OP;
    float *lcs = reinterpret_cast<float *>(a.ws + pl.off_lcs);
    float *dtp = reinterpret_cast<float *>(a.ws + pl.off_dtp);
    float *wgt = reinterpret_cast<float *>(a.ws + pl.off_wgt);
    OP *Hb = reinterpret_cast<OP *>(a.ws + pl.off_hb);
    float *St = reinterpret_cast<float *>(a.ws + pl.off_st);
    float *Lam = reinterpret_cast<float *>(a.ws + pl.off_lam);
    float *Scl = reinterpret_cast<float *>(a.ws + pl.off_scl);
    int *sgr = reinterpret_cast<int *>(a.ws + pl.off_sgr);
    const IO *x = static_cast<const IO *>(a.x);
    const IO *dt = static_cast<const IO *>(a.dt);
    const IO *Bm = static_cast<const IO *>(a.B);
    const IO *Cm = static_cast<const IO *>(a.C);
    IO *y = static_cast<IO *>(a.y);
    const int h = (int)pl.h, g = (int)pl.g;

    constexpr int HP = kGroupHeads<P>;
    const bool grouped = HP > 1 && group_heads((int)P, h / g) == HP;
    // the last chunk's own state is needed for the final state and for the
    // state after the last chunk
    const int keep_last = a.final_state != nullptr || a.states != nullptr;
    const bool seq = a.seq != nullptr;
    auto launch_state = [&](auto hp_c, auto seq_c) {
        constexpr int HPn = decltype(hp_c)::value;
        constexpr bool SQ = decltype(seq_c)::value;
        return launch_timed(&k_chunk_state<IO, P, N, HPn, SQ>,
                            dim3((unsigned)(pl.b * pl.nc * (h / HPn))),
                            dim3(Sp<IO, P, N, HPn>::NT), s, a.ev, kSlotState, x, Bm, dt, a.A,
                            a.dt_bias, a.softplus, a.dt_min, a.dt_max, lcs, dtp, wgt, St, Lam,
                            Scl, pl.l, h, g, pl.Q, pl.nc, pl.Qp, keep_last, a.seq, sgr, a.lw,
                            a.la);
    };
    hipError_t e;
    if (grouped)
        e = seq ? launch_state(std::integral_constant<int, HP>{}, std::true_type{})
                : launch_state(std::integral_constant<int, HP>{}, std::false_type{});
    else
        e = seq ? launch_state(std::integral_constant<int, 1>{}, std::true_type{})
                : launch_state(std::integral_constant<int, 1>{}, std::false_type{});
    if (e != hipSuccess) return e;

    const int64_t np4 = (int64_t)N * P / 4;
    const int64_t tot = pl.b * pl.h * np4;
    const int64_t scan_blocks = (tot + kThreads - 1) / kThreads;
    ImgArgs ia;
    ia.B = a.B;
    ia.C = a.C;
    ia.img = reinterpret_cast<f16 *>(a.ws + pl.off_img);
    ia.l = pl.l;
    ia.Q = pl.Q;
    ia.nc = pl.nc;
    ia.nsb = pl.nsb;
    ia.g = g;
    // bf16: one-head workgroups always copy (staging a whole block through
    // one or two waves' registers costs more registers than the output's
    // accumulators); head-sharing workgroups by the size rule
    const bool copy = sizeof(IO) == 2 && (!grouped || chunk_out_copy(h, g, P, N));
    ia.pieces = copy ? pl.b * pl.nc * g * pl.nsb * 2 * kT * (N / 8) : 0;
    if (keep_last)
        e = launch_timed(&k_state_scan<OP, IO, N, true>, dim3((unsigned)scan_blocks),
                         dim3(kThreads), s, a.ev, kSlotScan, St, Lam, Scl, a.init, Hb,
                         a.final_state, pl.b * pl.h, h, pl.nc, N, P, ia, a.states);
    else
        e = launch_timed(&k_state_scan<OP, IO, N, false>, dim3((unsigned)scan_blocks),
                         dim3(kThreads), s, a.ev, kSlotScan, St, Lam, Scl, a.init, Hb,
                         (float *)nullptr, pl.b * pl.h, h, pl.nc, N, P, ia, (float *)nullptr);
    if (e != hipSuccess) return e;

    auto launch_out = [&](auto hp_c, auto copy_c, auto seq_c) {
        constexpr int HPn = decltype(hp_c)::value;
        constexpr bool CP = decltype(copy_c)::value;
        constexpr bool SQ = decltype(seq_c)::value;
        return launch_timed(&k_chunk_out<IO, P, N, HPn, CP, SQ>,
                            dim3((unsigned)(pl.b * pl.nc * (h / HPn))),
                            dim3(Co<IO, P, N, HPn, CP>::NT), s, a.ev, kSlotOut, x, Bm, Cm, a.D,
                            lcs, dtp, wgt, Hb, y, pl.l, h, g, pl.Q, pl.nc, pl.Qp, ia.img, pl.nsb,
                            a.init != nullptr ? 1 : 0, sgr);
    };
    typedef std::integral_constant<int, 1> One;
    typedef std::integral_constant<int, HP> Grp;
    typedef std::true_type Yes;
    typedef std::false_type No;
    static_assert(sizeof(IO) == 4, "bf16 io has its own kernels (ssd_scan16.hpp)");
    (void)copy;
    if (grouped)
        return seq ? launch_out(Grp{}, No{}, Yes{}) : launch_out(Grp{}, No{}, No{});
    return seq ? launch_out(One{}, No{}, Yes{}) : launch_out(One{}, No{}, No{});
}

}  // namespace ssd
