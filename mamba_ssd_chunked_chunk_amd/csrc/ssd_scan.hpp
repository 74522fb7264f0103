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
// Rows are handled in blocks of T rows that never straddle a chunk boundary.
// With lcs_i the cumulative log2 decay inside a block (inclusive) and H the
// state entering the block:
//   y_i   = sum_{j<=i} (C_i . B_j) 2^(lcs_i - lcs_j) d_j x_j
//           + 2^lcs_i C_i^T H + D x_i                         (intra + read)
//   H'    = 2^lcs_last H + sum_j 2^(lcs_last - lcs_j) d_j B_j x_j^T  (write)
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

template <typename IO> struct Blk { static constexpr int T = 64; };
template <> struct Blk<float> { static constexpr int T = 32; };

// 8 consecutive elements of a row, loaded with vector loads.
template <typename IO> struct alignas(16) Row8v { IO e[8]; };

template <typename IO>
__device__ __forceinline__ Row8v<IO> ld_row8(const IO *p, bool valid) {
    Row8v<IO> v;
    if (valid) {
        v = *reinterpret_cast<const Row8v<IO> *>(p);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v.e[e] = from_f32<IO>(0.f);
    }
    return v;
}

template <typename IO>
__device__ __forceinline__ void st_row8(IO *dst, const Row8v<IO> &v) {
    *reinterpret_cast<Row8v<IO> *>(dst) = v;
}

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
    constexpr int T = Blk<IO>::T;
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
// 2. Chunk states and the serial pass over chunks.
//    One workgroup per (batch, segment, head, 32-row slice of the state).
//    The slice H[n0:n0+32, :] lives in MFMA accumulators for the whole
//    segment; each iteration stages up to 4 blocks (x^T and the weighted
//    B^T) in LDS and applies, block by block,
//        H <- 2^lcs_last H + (w B)^T x,  w_j = 2^(lcs_last - lcs_j) d_j.
//    Before the first block of every chunk the slice is written out as that
//    chunk's boundary state.  Segment 0 starts from init_state; later
//    segments start from zero and are corrected by k_seg_combine and in
//    k_chunk_out.
template <typename IO, int P, int N>
__global__ __launch_bounds__(256) void k_state_pass(
    const IO *__restrict__ x, const IO *__restrict__ Bm, const float *__restrict__ lcs,
    const float *__restrict__ dtp, const float *__restrict__ init, float *__restrict__ Hb,
    float *__restrict__ Eseg, float *__restrict__ Dlog, float *__restrict__ Lseg,
    float *__restrict__ final_state, int64_t l, int h, int g, int64_t Q, int64_t nc,
    int64_t Qp, int64_t cps, int64_t nseg) {
    typedef Mfma<IO> M;
    constexpr int T = Blk<IO>::T;
    constexpr int NW = 32;                  // state rows per workgroup
    constexpr int NSPLIT = N / NW;
    constexpr int SLAB = 4;                 // blocks per iteration
    constexpr int LDK = SLAB * T + M::PAD;  // LDS row: contraction axis
    constexpr int TILES = (NW / 16) * (P / 16);
    constexpr int TPW = (TILES + kWaves - 1) / kWaves;
    constexpr int XBLK = (T / 8) * (P / 8);
    constexpr int BBLK = (T / 8) * (NW / 8);
    __shared__ __attribute__((aligned(16))) IO XT[P * LDK];
    __shared__ __attribute__((aligned(16))) IO BT[NW * LDK];

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
    for (int i = 0; i < TPW; ++i) {
        acc[i] = zero4();
        const int ti = wave + kWaves * i;
        if (ti < TILES && seg == 0 && init) {
            const int tr = ti / (P / 16), tc = ti % (P / 16);
            const float *src = init + (b * h + hh) * NP +
                               (int64_t)(n0 + tr * 16 + 4 * (lane >> 4)) * P + tc * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = src[r * P];
        }
    }
    float logdec = 0.f;

    for (int64_t s0 = sb0; s0 < sb1; s0 += SLAB) {
        const int nb = (int)((sb1 - s0) < SLAB ? (sb1 - s0) : SLAB);
        // ---- stage x^T and (w B)^T of nb blocks
        for (int q = tid; q < nb * (XBLK + BBLK); q += kThreads) {
            const int j = q / (XBLK + BBLK);
            int rem = q % (XBLK + BBLK);
            const int64_t sb = s0 + j;
            const int64_t c = sb / nsb;
            const int64_t rpb = (sb % nsb) * T;  // padded row (in chunk) of block start
            if (rem < XBLK) {
                const int rb = rem / (P / 8), cb = rem % (P / 8);
                Row8v<IO> v[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t rp = rpb + rb * 8 + r, t = c * Q + rp;
                    const bool ok = rp < Q && t < l;
                    v[r] = ld_row8(x + ((b * l + (ok ? t : 0)) * h + hh) * P + cb * 8, ok);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Row8v<IO> o;
#pragma unroll
                    for (int r = 0; r < 8; ++r) o.e[r] = v[r].e[e];
                    st_row8(XT + (cb * 8 + e) * LDK + j * T + rb * 8, o);
                }
            } else {
                rem -= XBLK;
                const int rb = rem / (NW / 8), cb = rem % (NW / 8);
                const float last = lcs_bh[sb * T + T - 1];
                float w[8];
                Row8v<IO> v[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t R = sb * T + rb * 8 + r;
                    w[r] = exp2_fast(last - lcs_bh[R]) * dtp_bh[R];
                    const int64_t rp = rpb + rb * 8 + r, t = c * Q + rp;
                    const bool ok = rp < Q && t < l;
                    v[r] = ld_row8(Bm + ((b * l + (ok ? t : 0)) * g + gi) * N + n0 + cb * 8, ok);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Row8v<IO> o;
#pragma unroll
                    for (int r = 0; r < 8; ++r) o.e[r] = from_f32<IO>(to_f32(v[r].e[e]) * w[r]);
                    st_row8(BT + (cb * 8 + e) * LDK + j * T + rb * 8, o);
                }
            }
        }
        __syncthreads();
        // ---- apply the blocks in order
        for (int j = 0; j < nb; ++j) {
            const int64_t sb = s0 + j;
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
            const float lam = lcs_bh[sb * T + T - 1];
            const float decay = exp2_fast(lam);
            logdec += lam;
#pragma unroll
            for (int i = 0; i < TPW; ++i) acc[i] *= decay;
#pragma unroll
            for (int kk = 0; kk < T / M::K; ++kk) {
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int ti = wave + kWaves * i;
                    if (ti < TILES) {
                        const int tr = ti / (P / 16), tc = ti % (P / 16);
                        const auto fa = lds_frag(BT, LDK, tr * 16, j * T + kk * M::K, lane);
                        const auto fb = lds_frag(XT, LDK, tc * 16, j * T + kk * M::K, lane);
                        acc[i] = M::mma(fa, fb, acc[i]);
                    }
                }
            }
        }
        __syncthreads();
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
    f32x4 *E = reinterpret_cast<f32x4 *>(Eseg);
    auto slot = [&](int64_t k) { return ((b * nseg + k) * h + hh) * np4 + e4; };
    f32x4 H = E[slot(0)];
    for (int64_t k = 1; k < nseg; ++k) {
        const f32x4 Ek = E[slot(k)];
        E[slot(k - 1)] = H;
        H = exp2_fast(Lseg[pair * nseg + k]) * H + Ek;
    }
    if (final_state) reinterpret_cast<f32x4 *>(final_state)[pair * np4 + e4] = H;
}

// ----------------------------------------------------------------------------
// 4. Chunk output.  One workgroup per (batch, chunk, head); the blocks of the
//    chunk are taken in order with the running state H in MFMA accumulators
//    (fp32) and, as the bf16/fp32 operand copy H^T, in LDS.  Per block:
//      G^T = B C^T (causal tiles), P_ij = G_ij 2^(lcs_i - lcs_j) d_j (j <= i),
//      Y = 2^lcs_i (C H) + P x + D x,  then H <- 2^lcs_last H + (w B)^T x.
template <typename IO, int P, int N>
__global__ __launch_bounds__(256) void k_chunk_out(
    const IO *__restrict__ x, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ lcs, const float *__restrict__ dtp,
    const float *__restrict__ Hb, const float *__restrict__ Hin, const float *__restrict__ Dlog,
    IO *__restrict__ y, int64_t l, int h, int g, int64_t Q, int64_t nc, int64_t Qp,
    int64_t cps, int64_t nseg) {
    typedef Mfma<IO> M;
    constexpr int T = Blk<IO>::T;
    constexpr int LDN = N + M::PAD;  // rows with the state index contiguous
    constexpr int LDT = T + M::PAD;  // rows with the block-row index contiguous
    constexpr int BSZ = (T * LDN > T * LDT) ? T * LDN : T * LDT;
    constexpr int HTILES = (N / 16) * (P / 16);
    constexpr int HPW = (HTILES + kWaves - 1) / kWaves;
    constexpr int RT = T / 16;                       // row tiles per block
    constexpr int GTILES = RT * (RT + 1) / 2;        // causal tiles of P
    constexpr int GPW = (GTILES + kWaves - 1) / kWaves;
    constexpr int YTILES = RT * (P / 16);
    constexpr int YPW = (YTILES + kWaves - 1) / kWaves;
    constexpr int CBLK = (T / 8) * (N / 8);
    constexpr int XBLK = (T / 8) * (P / 8);
    __shared__ __attribute__((aligned(16))) IO Cs[T * LDN];   // C    [row][n]
    __shared__ __attribute__((aligned(16))) IO BP[BSZ];       // B [row][n], then P [i][j]
    __shared__ __attribute__((aligned(16))) IO BTw[N * LDT];  // (w B)^T [n][row]
    __shared__ __attribute__((aligned(16))) IO XT[P * LDT];   // x^T  [p][row]
    __shared__ __attribute__((aligned(16))) IO HT[P * LDN];   // H^T  [p][n]
    __shared__ float lcs_s[T];
    __shared__ float d_s[T];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

    // ---- state entering the chunk
    f32x4 accH[HPW];
    {
        const float *hb = Hb + ((b * nc + c) * h + hh) * NP;
        const float *hin = nullptr;
        float corr = 0.f;
        if (seg > 0) {
            hin = Hin + ((b * nseg + seg - 1) * h + hh) * NP;
            corr = exp2_fast(Dlog[(b * h + hh) * nc + c]);
        }
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            accH[i] = zero4();
            const int ti = wave + kWaves * i;
            if (ti < HTILES) {
                const int tr = ti / (P / 16), tc = ti % (P / 16);
                const int64_t off = (int64_t)(tr * 16 + 4 * (lane >> 4)) * P + tc * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = hb[off + r * P];
                    if (hin) v += corr * hin[off + r * P];
                    accH[i][r] = v;
                }
                lds_store4(HT + (tc * 16 + (lane & 15)) * LDN + tr * 16 + 4 * (lane >> 4), accH[i]);
            }
        }
    }

    const int64_t rows = (Q < l - c * Q) ? Q : (l - c * Q);  // valid rows of this chunk
    const int nblk = (int)((rows + T - 1) / T);

    for (int s = 0; s < nblk; ++s) {
        const int64_t rpb = (int64_t)s * T;  // padded row (in chunk) of the block start
        const float last = lcs_c[rpb + T - 1];
        // ---- stage C, B (natural), (w B)^T, x^T of this block
        for (int q = tid; q < 2 * CBLK + XBLK; q += kThreads) {
            if (q < 2 * CBLK) {
                const bool isB = q >= CBLK;
                const int qq = isB ? q - CBLK : q;
                const int rb = qq / (N / 8), cb = qq % (N / 8);
                const IO *src = isB ? Bm : Cm;
                Row8v<IO> v[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t rp = rpb + rb * 8 + r, t = c * Q + rp;
                    const bool ok = rp < Q && t < l;
                    v[r] = ld_row8(src + ((b * l + (ok ? t : 0)) * g + gi) * N + cb * 8, ok);
                }
                IO *nat = isB ? BP : Cs;
#pragma unroll
                for (int r = 0; r < 8; ++r) st_row8(nat + (rb * 8 + r) * LDN + cb * 8, v[r]);
                if (isB) {
                    float w[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int64_t R = rpb + rb * 8 + r;
                        w[r] = exp2_fast(last - lcs_c[R]) * dtp_c[R];
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        Row8v<IO> o;
#pragma unroll
                        for (int r = 0; r < 8; ++r) o.e[r] = from_f32<IO>(to_f32(v[r].e[e]) * w[r]);
                        st_row8(BTw + (cb * 8 + e) * LDT + rb * 8, o);
                    }
                }
            } else {
                const int qq = q - 2 * CBLK;
                const int rb = qq / (P / 8), cb = qq % (P / 8);
                Row8v<IO> v[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t rp = rpb + rb * 8 + r, t = c * Q + rp;
                    const bool ok = rp < Q && t < l;
                    v[r] = ld_row8(x + ((b * l + (ok ? t : 0)) * h + hh) * P + cb * 8, ok);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Row8v<IO> o;
#pragma unroll
                    for (int r = 0; r < 8; ++r) o.e[r] = v[r].e[e];
                    st_row8(XT + (cb * 8 + e) * LDT + rb * 8, o);
                }
            }
        }
        if (tid < T) {
            lcs_s[tid] = lcs_c[rpb + tid];
            d_s[tid] = dtp_c[rpb + tid];
        }
        __syncthreads();

        // ---- G^T tiles (rows j, columns i) and the masked, decayed P
        f32x4 pv[GPW];
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
            pv[u] = zero4();
            const int q = wave + kWaves * u;
            if (q < GTILES) {
                int it = 0;
                while ((it + 1) * (it + 2) / 2 <= q) ++it;
                const int jt = q - it * (it + 1) / 2;
                f32x4 gacc = zero4();
#pragma unroll
                for (int kk = 0; kk < N / M::K; ++kk) {
                    const auto fa = lds_frag(BP, LDN, jt * 16, kk * M::K, lane);
                    const auto fb = lds_frag(Cs, LDN, it * 16, kk * M::K, lane);
                    gacc = M::mma(fa, fb, gacc);
                }
                const int i = it * 16 + (lane & 15);
                const float li = lcs_s[i];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = jt * 16 + 4 * (lane >> 4) + r;
                    pv[u][r] = (j <= i) ? gacc[r] * exp2_fast(li - lcs_s[j]) * d_s[j] : 0.f;
                }
            }
        }
        __syncthreads();  // every read of B (natural) is done: BP becomes P
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
            const int q = wave + kWaves * u;
            if (q < GTILES) {
                int it = 0;
                while ((it + 1) * (it + 2) / 2 <= q) ++it;
                const int jt = q - it * (it + 1) / 2;
                lds_store4(BP + (it * 16 + (lane & 15)) * LDT + jt * 16 + 4 * (lane >> 4), pv[u]);
            }
        }
        // tiles above the diagonal that a contraction step of the next
        // product reaches are zero
        for (int it = wave; it < RT; it += kWaves) {
            const int kend = ((it + 1) * 16 + M::K - 1) / M::K * M::K;
            for (int jt = it + 1; jt * 16 < kend && jt < RT; ++jt)
                lds_store4(BP + (it * 16 + (lane & 15)) * LDT + jt * 16 + 4 * (lane >> 4), zero4());
        }
        __syncthreads();

        // ---- outputs of the block
#pragma unroll
        for (int u = 0; u < YPW; ++u) {
            const int ti = wave + kWaves * u;
            if (ti < YTILES) {
                const int it = ti / (P / 16), pt = ti % (P / 16);
                f32x4 ya = zero4();
#pragma unroll
                for (int kk = 0; kk < N / M::K; ++kk) {
                    const auto fa = lds_frag(Cs, LDN, it * 16, kk * M::K, lane);
                    const auto fb = lds_frag(HT, LDN, pt * 16, kk * M::K, lane);
                    ya = M::mma(fa, fb, ya);
                }
                const int i0 = it * 16 + 4 * (lane >> 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) ya[r] *= exp2_fast(lcs_s[i0 + r]);
                const int kend = ((it + 1) * 16 + M::K - 1) / M::K;
                for (int kk = 0; kk < kend; ++kk) {
                    const auto fa = lds_frag(BP, LDT, it * 16, kk * M::K, lane);
                    const auto fb = lds_frag(XT, LDT, pt * 16, kk * M::K, lane);
                    ya = M::mma(fa, fb, ya);
                }
                const int p = pt * 16 + (lane & 15);
                const f32x4 xv = lds_load4(XT + p * LDT + i0);
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
            const float decay = exp2_fast(last);
#pragma unroll
            for (int i = 0; i < HPW; ++i) accH[i] *= decay;
#pragma unroll
            for (int kk = 0; kk < T / M::K; ++kk) {
#pragma unroll
                for (int i = 0; i < HPW; ++i) {
                    const int ti = wave + kWaves * i;
                    if (ti < HTILES) {
                        const int tr = ti / (P / 16), tc = ti % (P / 16);
                        const auto fa = lds_frag(BTw, LDT, tr * 16, kk * M::K, lane);
                        const auto fb = lds_frag(XT, LDT, tc * 16, kk * M::K, lane);
                        accH[i] = M::mma(fa, fb, accH[i]);
                    }
                }
            }
            __syncthreads();  // every read of this block's operands is done
#pragma unroll
            for (int i = 0; i < HPW; ++i) {
                const int ti = wave + kWaves * i;
                if (ti < HTILES) {
                    const int tr = ti / (P / 16), tc = ti % (P / 16);
                    lds_store4(HT + (tc * 16 + (lane & 15)) * LDN + tr * 16 + 4 * (lane >> 4),
                               accH[i]);
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
