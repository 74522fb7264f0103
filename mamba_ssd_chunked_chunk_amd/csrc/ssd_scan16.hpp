// The chunked SSD scan for bf16 io on gfx950.
//
// The recurrence (nnterp guide, "Mamba-2" page, opening section)
//     h_t = exp(a_t) h_{t-1} + d_t B_t x_t^T,   y_t = C_t^T h_t + D x_t,
// a_t = A d_t, in the two-stage chunked form of the kongchang "Mamba2" page
// (chunk-scan entry): matrix products inside a chunk, one serial pass over
// chunks carrying the state, the state entering every chunk kept as one
// boundary-state tensor (nnterp, "The state after every token").
//
// Inside a chunk the rows go in blocks of T = 32 with a running state.  For
// block rows i, j (lcs the inclusive cumulative log2 decay inside the block,
// lam its total, w_j = 2^(lam - lcs_j) d_j the weight of row j in the state
// at the block's end):
//     y_i = sum_{j<=i} (C_i . B_j) 2^(lcs_i - lcs_j) d_j x_j
//           + 2^lcs_i C_i^T H + D x_i                           (read-out)
//     H  <- 2^lam H + B^T (w x)                                 (carry)
// Every exponent is <= 0 when A <= 0, and the j > i half of the scores is
// removed by a select, so no inf * 0 reaches a result.
//
// Matrix-core operands.  The products run on v_mfma_f32_16x16x32_bf16 with
// fp32 accumulation.  The inputs x, B and C are bf16 and enter the products
// exactly as they are.  Every operand made inside the scan (the carried
// state H, the masked scores with the skip term on their diagonal, and the
// decay-weighted x) is an fp32 value v written as two bf16 terms,
// hi = bf16(v) and lo = bf16(v - hi), and multiplied as two products: 16
// significant bits and fp32's exponent range, so any finite bf16 input is
// handled.
//
// Launch sequence on one stream:
//   1. k_state16  every chunk's own state from zero (all chunks in
//                 parallel), stored as fp16 times a power of two per
//                 (batch, chunk, head), with its largest magnitude and the
//                 chunk's total log2 decay
//   2. k_scan16   the serial pass over chunks: H_{c+1} = 2^L_c H_c + S_c in
//                 fp32; boundary states stored as fp16 times a power of two
//                 taken from a running bound on their magnitude; the final
//                 state and the state after every chunk in fp32
//   3. k_out16    the chunk output from the boundary states
// The chunk-state pass and the chunk output are persistent: each workgroup
// walks the 32-row blocks of a fixed list of (batch, chunk, heads) items
// back to back, the copy of the next block (which may open the next item)
// in flight while the current one is computed.  Both compute the per-row
// time step, cumulative decay and weights of each block from the raw time
// steps with the same code, so they agree bit for bit.
#pragma once

#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {
namespace s16 {

constexpr int T = 32;  // rows per block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// An fp32 operand as two bf16 terms.
struct HL {
    bf16x8 hi, lo;
};
__device__ __forceinline__ HL split8(const float (&v)[8]) {
    HL o;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 h = __builtin_convertvector((f32x2{v[e], v[e + 1]}), bf16x2);
        const f32x2 r{v[e] - (float)h[0], v[e + 1] - (float)h[1]};
        const bf16x2 q = __builtin_convertvector(r, bf16x2);
        o.hi[e] = h[0];
        o.hi[e + 1] = h[1];
        o.lo[e] = q[0];
        o.lo[e + 1] = q[1];
    }
    return o;
}
// Two accumulator tiles (contraction blocks 0..15 and 16..31 of a 32-block)
// as one operand in the k convention of ssd_device.hpp.
__device__ __forceinline__ HL split_acc(const f32x4 &t0, const f32x4 &t1) {
    const float v[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    return split8(v);
}
// A raw operand fragment (8 bf16 as two 8-byte halves) from LDS bits.
__device__ __forceinline__ bf16x8 as_bf16x8(const f16x4 &a, const f16x4 &b) {
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(bf16x8, u32x4{ua[0], ua[1], ub[0], ub[1]});
}
// Bit reinterpretation of one 32-bit value.  Always through these by-value
// helpers: __builtin_bit_cast applied directly to an element of an
// ext_vector_type value reads element 0 whatever the index (the compiler
// takes the vector's address), so vector elements are first copied into a
// scalar parameter.
__device__ __forceinline__ float as_f32(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ uint32_t as_u32(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// ------------------------------------------------------------ shapes ----
// HP heads of one group per workgroup (they share the staged B and C),
// WPH waves per head, each owning PW head_dim columns of its head.
template <int P, int N, int HP> struct Shape {
    static constexpr int WPH = P >= 64 ? P / 32 : 1;
    static constexpr int PW = P / WPH;
    static constexpr int CPW = PW / 16;  // column tiles per wave
    static constexpr int W = HP * WPH, NT = 64 * W;
    static constexpr int RT = N / 16;  // state row tiles
    static constexpr int NB = N / 32;  // 32-blocks of the state index
    static constexpr int XE = HP * T * P;  // x elements of a block (all heads)
    static constexpr int BE = T * N;       // B (or C) elements of a block
    // 16-byte copies of a block (x, B, and for the chunk output C), in
    // wave instructions of 64 copies, and per wave (rounded up: waves past
    // the last instruction copy into a spare slot from an empty source)
    static constexpr int XI = XE / 8 / 64, BI = BE / 8 / 64;
    template <bool WITH_C> static constexpr int ninst() { return XI + BI * (WITH_C ? 2 : 1); }
    template <bool WITH_C> static constexpr int per_wave() { return (ninst<WITH_C>() + W - 1) / W; }
    // y stores per lane and block
    static constexpr int NS = CPW % 2 == 0 ? CPW : 2 * CPW;
    static_assert(XE % 512 == 0 && BE % 512 == 0, "whole copy instructions");
};

// Raw bf16 x in LDS: row r of a head holds head_dim elements in 16-byte
// chunks, chunk k at position k ^ xsw(r).
template <int P> __device__ __forceinline__ int xsw(int r) {
    return ((((r >> 1) & 3) << 2)) & (P / 8 - 1);
}
template <int P> __device__ __forceinline__ int xsw_at(int r, int col) {
    return r * P + (((col >> 3) ^ xsw<P>(r)) << 3) + (col & 7);
}

// head_dim column of row rho (0..15) of a wave's column tile u: tiles go
// in pairs that interleave in groups of 4 columns, so that a lane's output
// rows of the two tiles are 8 consecutive columns.
template <int CPW> __device__ __forceinline__ int col_of(int u, int rho) {
    if constexpr (CPW % 2 == 0)
        return 32 * (u >> 1) + 8 * (rho >> 2) + 4 * (u & 1) + (rho & 3);
    else
        return 16 * u + rho;
}

// k-major x fragment of column tile u (contraction index = block row).
template <int CPW, int P>
__device__ __forceinline__ bf16x8 x_frag(const f16 *Xs, int c0, int u, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int col = c0 + col_of<CPW>(u, 4 * (j & 3));
    const int ra = 4 * g + (j >> 2), rb = 16 + ra;
    const f16x4 a = __builtin_bit_cast(
        f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(Xs + xsw_at<P>(ra, col))));
    const f16x4 b = __builtin_bit_cast(
        f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(Xs + xsw_at<P>(rb, col))));
    return as_bf16x8(a, b);
}
// Rows of a swizzled [T][N] matrix in the k convention (contraction over
// columns kb..kb+31): lane l gets row row0 + (l & 15).
template <int N>
__device__ __forceinline__ bf16x8 rows_frag(const f16 *M, int row0, int kb, int lane) {
    typedef Swz<f16, N> S;
    const int r = row0 + (lane & 15), g = lane >> 4;
    const f16x4 a = *reinterpret_cast<const f16x4 *>(M + S::at(r, kb + 4 * g));
    const f16x4 b = *reinterpret_cast<const f16x4 *>(M + S::at(r, kb + 16 + 4 * g));
    return as_bf16x8(a, b);
}
// k-major fragment (contraction over the 32 rows) of columns c0..c0+15 of a
// swizzled [T][N] matrix.
template <int N>
__device__ __forceinline__ bf16x8 kmajor_frag(const f16 *M, int c0, int lane) {
    typedef Swz<f16, N> S;
    const int g = lane >> 4, j = lane & 15;
    const f16 *pa = M + S::at(4 * g + (j >> 2), c0 + 4 * (j & 3));
    const f16 *pb = M + S::at(16 + 4 * g + (j >> 2), c0 + 4 * (j & 3));
    const f16x4 a =
        __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pa));
    const f16x4 b =
        __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pb));
    return as_bf16x8(a, b);
}
// The k-major x fragment weighted row by row (rows 4g + r and 16 + 4g + r
// of lane group g) by w, as two bf16 terms.
__device__ __forceinline__ HL xw_split(const bf16x8 &xf, int lane, const float *w) {
    const int g = lane >> 4;
    const f32x4 wa = *reinterpret_cast<const f32x4 *>(w + 4 * g);
    const f32x4 wb = *reinterpret_cast<const f32x4 *>(w + 16 + 4 * g);
    const u32x4 xb = __builtin_bit_cast(u32x4, xf);
    const float v[8] = {bf16_lo(xb[0]) * wa[0], bf16_hi(xb[0]) * wa[1],
                        bf16_lo(xb[1]) * wa[2], bf16_hi(xb[1]) * wa[3],
                        bf16_lo(xb[2]) * wb[0], bf16_hi(xb[2]) * wb[1],
                        bf16_lo(xb[3]) * wb[2], bf16_hi(xb[3]) * wb[3]};
    return split8(v);
}

// -------------------------------------------------- per-row values ----
// Per-row values of one block of one head, kept by each wave for its own
// head in LDS (pairs (i, i + 16) interleaved where a lane reads both rows it
// owns at once).
struct alignas(16) Rows {
    float lcs[T];  // cumulative log2 decay inside the block (inclusive)
    float d[T];    // processed time step (0 past the chunk's end)
    float w[T];    // 2^(lcs_31 - lcs_j) d_j: weight in the state at the block's end
    float a2[T];   // 2^(lcs_i - lcs_15), pairs (i, i + 16) at 2 (i % 16)
    float l2[T];   // lcs_i in the same pairs
    float bw[T];   // 2^(lcs_15 - lcs_j) d_j
    int seg[T];    // packed sequences: the last row <= i of the block that starts a
                   // new document, or -1
};
__device__ __forceinline__ int row_pair(int r) { return 2 * (r & 15) + (r >> 4); }


// Raw per-row inputs of one block for one head: lane l holds row l & 31
// (the two halves of a wave hold the same rows).
struct RowIn {
    float dt;
    int rst;  // packed sequences: the row starts a new document
};

// Where one head's rows of a chunk live.
struct RowSrc {
    const bf16 *dt;      // the chunk's first row, this head (rows `h` elements apart)
    const int32_t *seq;  // the sequence's document indices (packed sequences), or null
    int64_t t0, l;       // the chunk's first token, the sequence length
    int h;               // heads
    int rows;            // valid rows of the chunk
};

// Loads block k's raw rows: one vector memory operation per lane (three
// with packed sequences).  Rows past the chunk's end read as zero.
template <bool SEQ>
__device__ __forceinline__ void rows_load(RowIn &f, const RowSrc &rs, int k, int lane) {
    const int r = lane & 31;
    int valid = rs.rows - k * T;
    valid = valid < 0 ? 0 : (valid > T ? T : valid);
    const Rsrc rd = make_rsrc(rs.dt + (int64_t)(valid > 0 ? k * T : 0) * rs.h,
                              (int64_t)valid * rs.h * 2);
    const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(rd, (uint32_t)(r * rs.h * 2), 0, 0);
    f.dt = __builtin_bit_cast(float, (uint32_t)v << 16);
    f.rst = 0;
    if constexpr (SEQ) {
        // a row whose document index differs from the previous token's
        // starts from a zero state (token 0 starts from the initial state)
        const int64_t t = rs.t0 + (int64_t)k * T + r;
        const Rsrc rq = make_rsrc(rs.seq, rs.l * 4);
        const int cur = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, (uint32_t)(t * 4), 0, 0);
        const int prv =
            (int)__builtin_amdgcn_raw_buffer_load_b32(rq, (uint32_t)(t * 4) - 4u, 0, 0);
        f.rst = (k * T + r < rs.rows && t > 0) ? (cur != prv) : 0;
    }
}
template <bool SEQ> constexpr int kRowOps = SEQ ? 3 : 1;

// The block's per-row values from its raw rows, written to R (lanes 0..31)
// by the wave that owns the head; returns the block's log2 decay as seen
// by the state carry (-inf when a document starts inside the block:
// nothing before the reset reaches the block's end).
template <bool SEQ>
__device__ __forceinline__ float rows_prep(Rows &R, const RowIn &f, float a2, float bias,
                                           int softplus, float lo, float hi, int k, int rows,
                                           int lane) {
    const int r = lane & 31;
    const bool valid = k * T + r < rows;
    const float d = valid ? time_step(f.dt, bias, softplus, lo, hi) : 0.f;
    float a = a2 * d;
    // inclusive prefix sum over the block's 32 rows (each 32-lane half)
#pragma unroll
    for (int off = 1; off < T; off <<= 1) {
        const float v = __shfl_up(a, off, T);
        if (r >= off) a += v;
    }
    const float last = __shfl(a, T - 1, T);
    const float l15 = __shfl(a, 15, T);
    float w = exp2_fast(last - a) * d;
    float lam = last;
    int seg = -1;
    if constexpr (SEQ) {
        const uint32_t m = (uint32_t)(__ballot(f.rst != 0) >> (lane & 32));
        if (m) {
            if (r < 31 - __builtin_clz(m)) w = 0.f;
            lam = -INFINITY;
        }
        const uint32_t mr = m & ((2u << r) - 1u);
        seg = mr ? 31 - __builtin_clz(mr) : -1;
    }
    if (lane < 32) {
        R.lcs[r] = a;
        R.d[r] = d;
        R.w[r] = w;
        R.a2[row_pair(r)] = exp2_fast(a - l15);
        R.l2[row_pair(r)] = a;
        R.bw[r] = exp2_fast(l15 - a) * d;
        if constexpr (SEQ) R.seg[r] = seg;
    }
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lam)));
}

// Power-of-two scale of an fp16 store: m (>= the largest magnitude) times
// inv lands below 2^15 (fp16's largest finite value is about 2^16); scale =
// 1 / inv.  Magnitudes below 2^-100 take the scale of 2^-100.
__device__ __forceinline__ int scale_exp(float m) {
    int ex = -100;
    if (m >= 0x1p-100f) frexpf(m, &ex);  // m = f 2^ex, f in [0.5, 1)
    return ex;
}

// --------------------------------------------------- work items ----
// Item = (batch, chunk, HP consecutive heads of one group), heads fastest.
// Workgroups take items round robin from a worker index that keeps
// consecutive indices on one XCD (xcd_item), so the heads of one (batch,
// chunk) meet in that XCD's L2.
struct Item {
    int64_t b, c;
    int hh0, gi, rows, nblk;
    int64_t t0;
    bool live;
};
__device__ __forceinline__ Item decode_item(int64_t item, int64_t items, int64_t nc_items,
                                            int hpg_items, int h, int g, int64_t l, int64_t Q,
                                            int HP) {
    Item it;
    it.live = item < items;
    const int64_t q = it.live ? item : 0;
    const int hq = (int)(q % hpg_items);
    const int64_t bc = q / hpg_items;
    it.c = bc % nc_items;
    it.b = bc / nc_items;
    it.hh0 = hq * HP;
    it.gi = it.hh0 / (h / g);
    it.t0 = it.c * Q;
    const int64_t rem = l - it.t0;
    it.rows = (int)(rem < Q ? rem : Q);
    it.nblk = it.live ? (it.rows + T - 1) / T : 0;
    return it;
}

// The 16-byte copies of one block into LDS buffer `buf` ([x of each head |
// B | C], C only WITH_C): wave instruction q of the block copies 64
// consecutive slots;
// each lane fetches the 16-byte source chunk its (swizzled) slot holds.
// Rows past the chunk's end read as zeros.  Each wave issues exactly
// per_wave<WITH_C>() copies (the spare slot takes the rest).
template <int P, int N, int HP, bool WITH_C>
__device__ __forceinline__ void block_copy(f16 *buf, f16 *spare, const bf16 *x, const bf16 *B,
                                           const bf16 *C, int64_t xs, int64_t bs, int valid,
                                           int wave, int lane) {
    typedef Shape<P, N, HP> K;
    constexpr int CH = P / 8, CB = N / 8;
    const Rsrc rx = make_rsrc(x, (int64_t)valid * xs * 2);
    const Rsrc rb = make_rsrc(B, (int64_t)valid * bs * 2);
    const Rsrc rc = make_rsrc(WITH_C ? C : B, WITH_C ? (int64_t)valid * bs * 2 : 0);
#pragma unroll
    for (int j = 0; j < K::template per_wave<WITH_C>(); ++j) {
        const int q = wave + j * K::W;
        if (q < K::XI) {
            const int s = q * 64 + lane;
            const int hs = s / (T * CH), rem = s % (T * CH), r = rem / CH, kk = rem % CH;
            const uint32_t off =
                (uint32_t)(r * xs + hs * P + ((kk ^ xsw<P>(r)) << 3)) * 2u;
            lds_copy16(rx, (lds_void *)(buf + q * 512), off);
        } else if (q < K::XI + K::BI * (WITH_C ? 2 : 1)) {
            const int qb = q - K::XI;
            const bool isC = WITH_C && qb >= K::BI;
            const int s = (isC ? qb - K::BI : qb) * 64 + lane;
            const int r = s / CB, kk = s % CB;
            const uint32_t off = (uint32_t)(r * bs + ((kk ^ Swz<f16, N>::f(r)) << 3)) * 2u;
            lds_copy16(isC ? rc : rb, (lds_void *)(buf + q * 512), off);
        } else {
            lds_copy16(rc, (lds_void *)spare, 0u);
        }
    }
}

// ----------------------------------------------------------------------------
// 1. Chunk states: every item's chunk from a zero state,
//        S <- 2^lam S + B^T (w x)   per block,
//    each wave holding its head_dim columns of its head's state (all
//    state_dim rows) in MFMA accumulators.  At an item's end the state is
//    stored transposed ([head_dim][state_dim]) as fp16 times 2^(15 - e),
//    e the exponent of the head's largest magnitude m (written as Smax),
//    with the chunk's total log2 decay (Lam); chunk-0 items also write the
//    largest magnitude of the initial state of their heads (Imax).
template <int P, int N, int HP, bool SEQ>
__global__ __launch_bounds__((Shape<P, N, HP>::NT), 3) void k_state16(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ dt,
    const float *__restrict__ A, const float *__restrict__ dt_bias, int softplus, float dt_min,
    float dt_max, const int32_t *__restrict__ seq, const float *__restrict__ init,
    f16 *__restrict__ St, float *__restrict__ Smax, float *__restrict__ Lam,
    float *__restrict__ Imax, int64_t l, int h, int g, int64_t Q, int64_t nc, int64_t nc_items,
    int64_t items) {
    typedef Shape<P, N, HP> K;
    constexpr int BUF = K::XE + K::BE, CPW = K::CPW, RT = K::RT, WPH = K::WPH;
    __shared__ __attribute__((aligned(16))) f16 lds0[BUF];
    __shared__ __attribute__((aligned(16))) f16 lds1[BUF];
    __shared__ __attribute__((aligned(16))) f16 spare[512];
    __shared__ Rows rows0[K::W];
    __shared__ Rows rows1[K::W];
    __shared__ float wmax[K::W], wimax[K::W];

    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int hs = wave / WPH, c0 = (wave % WPH) * K::PW;
    const int64_t G = gridDim.x;
    const int64_t v = xcd_item(blockIdx.x, G);
    const int hpg = h / HP;
    const int64_t NP = (int64_t)N * P;
    const int64_t xs = (int64_t)h * P, bs = (int64_t)g * N;

    int64_t item = v;
    Item it = decode_item(item, items, nc_items, hpg, h, g, l, Q, HP);
    if (!it.live) return;

    auto rsrc_of = [&](const Item &q) {
        RowSrc rs;
        rs.dt = dt + (q.b * l + q.t0) * h + q.hh0 + hs;
        rs.seq = SEQ ? seq + q.b * l : nullptr;
        rs.t0 = q.t0;
        rs.l = l;
        rs.h = h;
        rs.rows = q.rows;
        return rs;
    };
    auto copy = [&](f16 *buf, const Item &q, int k) {
        int valid = q.live ? q.rows - k * T : 0;
        valid = valid < 0 ? 0 : (valid > T ? T : valid);
        const int64_t r0 = valid > 0 ? q.t0 + (int64_t)k * T : 0;
        block_copy<P, N, HP, false>(buf, spare, x + ((q.b * l + r0) * h + q.hh0) * P,
                                    Bm + ((q.b * l + r0) * g + q.gi) * N, nullptr, xs, bs, valid,
                                    wave, lane);
    };

    float a2 = A[it.hh0 + hs] * kLog2e;
    float bias = dt_bias ? dt_bias[it.hh0 + hs] : 0.f;
    RowSrc rs = rsrc_of(it);

    // prologue: block 0 of the first item
    RowIn ri;
    rows_load<SEQ>(ri, rs, 0, lane);
    copy(lds0, it, 0);
    vm_wait<0>();
    float lam = rows_prep<SEQ>(rows0[wave], ri, a2, bias, softplus, dt_min, dt_max, 0, it.rows,
                               lane);

    f32x4 acc[CPW * RT];
#pragma unroll
    for (int t = 0; t < CPW * RT; ++t) acc[t] = zero4();
    float logdec = 0.f;
    int k = 0;  // block of the current item

    // Stores the finished item's state (its wave maxima are in wmax).
    auto finish = [&](const Item &q) {
        float m = 0.f, mi = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < WPH; ++w2) {
            m = fmaxf(m, wmax[hs * WPH + w2]);
            mi = fmaxf(mi, wimax[hs * WPH + w2]);
        }
        const int ex = scale_exp(m);
        const float inv = ldexpf(1.f, 15 - ex);
        const int hh = q.hh0 + hs;
        f16 *dst = St + ((q.b * nc + q.c) * h + hh) * NP;
#pragma unroll
        for (int u = 0; u < CPW; ++u)
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) {
                const f32x4 s = acc[u * RT + tr] * inv;
                *reinterpret_cast<f16x4 *>(dst + (c0 + col_of<CPW>(u, lane & 15)) * N + tr * 16 +
                                           4 * (lane >> 4)) =
                    f16x4{(f16)s[0], (f16)s[1], (f16)s[2], (f16)s[3]};
            }
        if (c0 == 0 && lane == 0) {
            Smax[(q.b * h + hh) * nc + q.c] = m;
            Lam[(q.b * h + hh) * nc + q.c] = logdec;
            if (init && q.c == 0) Imax[q.b * h + hh] = mi;
        }
    };
    // The wave's largest magnitudes of the finished item (and of its heads'
    // initial state on chunk-0 items), for finish() after the next barrier.
    auto wave_max = [&](const Item &q) {
        float m = 0.f;
#pragma unroll
        for (int t = 0; t < CPW * RT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(acc[t][e]));
        float mi = 0.f;
        if (init && q.c == 0) {
            const float *src = init + (q.b * h + q.hh0 + hs) * NP;
            const int part = wave % WPH;
            for (int64_t e = (int64_t)(part * 64 + lane) * 4; e < NP; e += 64 * WPH * 4) {
                const f32x4 iv = *reinterpret_cast<const f32x4 *>(src + e);
                mi = fmaxf(mi, fmaxf(fmaxf(fabsf(iv[0]), fabsf(iv[1])),
                                     fmaxf(fabsf(iv[2]), fabsf(iv[3]))));
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            m = fmaxf(m, __shfl_xor(m, off, 64));
            mi = fmaxf(mi, __shfl_xor(mi, off, 64));
        }
        if (lane == 0) {
            wmax[wave] = m;
            wimax[wave] = mi;
        }
    };

    // One block: the state decays by the block's total and takes its rows.
    auto compute = [&](const f16 *buf, const Rows &R, float lm) {
        const float dec = exp2_fast(lm);
#pragma unroll
        for (int t = 0; t < CPW * RT; ++t) acc[t] *= dec;
        const f16 *Xs = buf + hs * T * P;
        const f16 *Bs = buf + K::XE;
        HL xw[CPW];
#pragma unroll
        for (int u = 0; u < CPW; ++u) xw[u] = xw_split(x_frag<CPW, P>(Xs, c0, u, lane), lane, R.w);
#pragma unroll
        for (int tr = 0; tr < RT; ++tr) {
            const bf16x8 bt = kmajor_frag<N>(Bs, tr * 16, lane);
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                acc[u * RT + tr] = mma(bt, xw[u].hi, acc[u * RT + tr]);
                acc[u * RT + tr] = mma(bt, xw[u].lo, acc[u * RT + tr]);
            }
        }
    };

    // Blocks go in pairs (LDS buffer 0, then 1) so that every access names
    // its buffer statically.  At the top of a half: the block's copy and
    // rows have landed; the barrier also tells that every wave is done with
    // the other buffer, into which the next block is then copied.
    bool pending = false;  // an item ended with the previous block
    Item done = it;
    for (;;) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f16 *const bk = half == 0 ? lds0 : lds1;
            f16 *const bn = half == 0 ? lds1 : lds0;
            Rows &Rk = half == 0 ? rows0[wave] : rows1[wave];
            Rows &Rn = half == 0 ? rows1[wave] : rows0[wave];
            lds_barrier();
            if (pending) {
                finish(done);
#pragma unroll
                for (int t = 0; t < CPW * RT; ++t) acc[t] = zero4();
                logdec = 0.f;
                pending = false;
            }
            // the next block: this item's next, or the next item's first
            Item nx = it;
            int kn = k + 1;
            if (kn >= it.nblk) {
                nx = decode_item(item + G, items, nc_items, hpg, h, g, l, Q, HP);
                kn = 0;
            }
            const RowSrc rsn = nx.live ? rsrc_of(nx) : rs;
            RowIn rn;
            copy(bn, nx, kn);
            rows_load<SEQ>(rn, rsn, nx.live ? kn : 1 << 20, lane);
            issue_fence();
            compute(bk, Rk, lam);
            logdec += lam;
            if (k + 1 >= it.nblk) {
                wave_max(it);
                pending = true;
                done = it;
            }
            if (!nx.live) {
                lds_barrier();
                finish(done);
                vm_wait<0>();
                return;
            }
            vm_wait<0>();
            if (kn == 0) {
                item += G;
                it = nx;
                rs = rsn;
                a2 = A[it.hh0 + hs] * kLog2e;
                bias = dt_bias ? dt_bias[it.hh0 + hs] : 0.f;
            }
            k = kn;
            lam = rows_prep<SEQ>(Rn, rn, a2, bias, softplus, dt_min, dt_max, k, it.rows, lane);
        }
    }
}

// ----------------------------------------------------------------------------
// 2. State scan: the serial pass over chunks,
//        H_0 = init (or 0),   H_{c+1} = 2^L_c H_c + S_c   (fp32),
//    with S_c (fp16 times 2^(e_c - 15), e_c = scale_exp(Smax)) and L_c from
//    k_state16.  Chunk c's boundary state H_c is stored transposed
//    ([head_dim][state_dim]) as fp16 times 2^(15 - E_c), E_c = scale_exp(M_c)
//    for the running bound M_0 = max |init|, M_{c+1} = 2^L_c M_c + max|S_c|
//    >= max |H_{c+1}| (every thread of a (batch, head) computes the same
//    bound, so the scale needs no exchange); 2^(E_c - 15) goes to Hs.  The
//    state after the last chunk is the final state ([state_dim][head_dim],
//    fp32).  One thread per 4 consecutive state elements, as ScanTile in
//    ssd_scan.hpp lays them out; chunk states are loaded 8 chunks ahead.
template <int N, bool ROWS>
__global__ __launch_bounds__(256) void k_scan16(
    const f16 *__restrict__ St, const float *__restrict__ Smax, const float *__restrict__ Lam,
    const float *__restrict__ Imax, const float *__restrict__ init, f16 *__restrict__ Hb,
    float *__restrict__ Hs, float *__restrict__ final_state, int64_t bh, int h, int64_t nc,
    int n, int p, float *__restrict__ states) {
    constexpr int G8 = 8;
    __shared__ __attribute__((aligned(16))) float lds[4 * 256];
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t np4 = (int64_t)n * p / 4;
    // threads past the last element stay for the barriers of the row stores
    const bool live = idx < bh * np4;
    if (!ROWS) states = final_state = nullptr;
    if (!live && !ROWS) return;
    const int64_t ie = live ? idx : bh * np4 - 1;
    const ScanTile st(n, p);
    const int64_t tile = ie / st.TT;
    const int loc = (int)(ie % st.TT);
    const int64_t tpp = (int64_t)(n / st.R) * (p / st.Cc);
    const int64_t pair = tile / tpp, tip = tile % tpp;
    const int row0 = (int)(tip % (n / st.R)) * st.R, col0 = (int)(tip / (n / st.R)) * st.Cc;
    const int64_t b = pair / h, hh = pair % h;
    const int64_t n0 = row0 + (loc % (st.R / 4)) * 4, pc = col0 + loc / (st.R / 4);
    const int64_t e4 = (pc * n + n0) / 4;
    // the (batch, head)'s first thread writes the boundary states' scales
    const bool lead = live && ie % np4 == 0;
    f32x4 H = zero4();
    float M = 0.f;
    if (init) {
        const float *src = init + pair * (int64_t)n * p + n0 * p + pc;
#pragma unroll
        for (int e = 0; e < 4; ++e) H[e] = src[e * p];
        M = Imax[pair];
    }
    const int64_t cstride = (int64_t)h * np4;
    const f16x4 *S16 = reinterpret_cast<const f16x4 *>(St) + (b * nc * h + hh) * np4 + e4;
    f16x4 *dst = reinterpret_cast<f16x4 *>(Hb) + (b * nc * h + hh) * np4 + e4;
    const float *L = Lam + pair * nc;
    const float *Sm = Smax + pair * nc;
    float *hsc = Hs + pair * nc;
    const int64_t ns = (final_state || states) ? nc : nc - 1;
    const int64_t klast = ns > 0 ? ns - 1 : 0;
    for (int64_t k0 = 0; k0 < nc; k0 += G8) {
        f16x4 Sh[G8];
        float Lk[G8], Mk[G8];
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int64_t k = k0 + u < klast ? k0 + u : klast;
            Sh[u] = S16[k * cstride];
            Lk[u] = L[k];
            Mk[u] = Sm[k];
        }
#pragma unroll
        for (int u = 0; u < G8; ++u) {
            const int64_t c = k0 + u;
            // chunk 0's boundary state is stored only for a given initial
            // state (the chunk output takes zeros otherwise)
            if (live && c < nc && (c > 0 || init)) {
                const int ex = scale_exp(M);
                const f32x4 hv = H * ldexpf(1.f, 15 - ex);
                dst[c * cstride] = f16x4{(f16)hv[0], (f16)hv[1], (f16)hv[2], (f16)hv[3]};
                if (lead) hsc[c] = ldexpf(1.f, ex - 15);
            }
            if (c < ns) {
                const float sc = ldexpf(1.f, scale_exp(Mk[u]) - 15);
                const f32x4 S = f32x4{(float)Sh[u][0], (float)Sh[u][1], (float)Sh[u][2],
                                      (float)Sh[u][3]} * sc;
                const float dec = exp2_fast(Lk[u]);
                H = dec * H + S;
                M = dec * M + Mk[u];
            }
            if (ROWS && states && c < nc)
                store_state_rows(lds, H, st, live,
                                 states + ((b * nc + c) * h + hh) * (int64_t)n * p, row0, col0, p);
        }
    }
    if (ROWS && final_state)
        store_state_rows(lds, H, st, live, final_state + pair * (int64_t)n * p, row0, col0, p);
}

// ----------------------------------------------------------------------------
// 3. Chunk output: every item's chunk from its boundary state.  Each wave
//    seeds its head_dim columns of the running state H (all state_dim rows,
//    MFMA accumulators) from the stored boundary state and walks the chunk's
//    blocks; per block:
//      G^T = B C^T on the 3 causal 16 x 16 tiles, and
//      P_ij = G_ij 2^(lcs_i - lcs_j) d_j (j <= i) in registers;
//      y^T = 2^lcs_i (H^T C^T) + x^T (P + D I)^T (the skip term on the
//            scores' diagonal), stored straight from the accumulators;
//      H <- 2^lcs_last H + B^T (w x)  (except after the item's last block).
//    The scores and the read-out share the C fragments.  The decay factor
//    of P is taken as a_i b_j with a_i = 2^(lcs_i - lcs_15) and
//    b_j = 2^(lcs_15 - lcs_j) d_j when the block's total log2 decay is above
//    -kSplit (every factor then stays inside fp32's normal range); otherwise
//    as one exponential per element.  In an item's last block, once the
//    read-out has taken H, the next item's boundary state is requested into
//    the same registers.
constexpr float kSplit = 60.f;

template <int P, int N, int HP, bool SEQ>
__global__ __launch_bounds__((Shape<P, N, HP>::NT), 2) void k_out16(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const bf16 *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ D,
    const float *__restrict__ dt_bias, int softplus, float dt_min, float dt_max,
    const int32_t *__restrict__ seq, const f16 *__restrict__ Hb, const float *__restrict__ Hs,
    bf16 *__restrict__ y, int64_t l, int h, int g, int64_t Q, int64_t nc, int has_init,
    int64_t items) {
    typedef Shape<P, N, HP> K;
    constexpr int BUF = K::XE + 2 * K::BE, CPW = K::CPW, RT = K::RT, WPH = K::WPH,
                  NB = K::NB, NS = K::NS;
    __shared__ __attribute__((aligned(16))) f16 lds0[BUF];
    __shared__ __attribute__((aligned(16))) f16 lds1[BUF];
    __shared__ __attribute__((aligned(16))) f16 spare[512];
    __shared__ Rows rows0[K::W];
    __shared__ Rows rows1[K::W];

    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int lg = lane >> 4, li = lane & 15;
    const int hs = wave / WPH, c0 = (wave % WPH) * K::PW;
    const int64_t G = gridDim.x;
    const int64_t v = xcd_item(blockIdx.x, G);
    const int hpg = h / HP;
    const int64_t NP = (int64_t)N * P;
    const int64_t xs = (int64_t)h * P, bs = (int64_t)g * N;

    int64_t item = v;
    Item it = decode_item(item, items, nc, hpg, h, g, l, Q, HP);
    if (!it.live) return;

    auto rsrc_of = [&](const Item &q) {
        RowSrc rs;
        rs.dt = dt + (q.b * l + q.t0) * h + q.hh0 + hs;
        rs.seq = SEQ ? seq + q.b * l : nullptr;
        rs.t0 = q.t0;
        rs.l = l;
        rs.h = h;
        rs.rows = q.rows;
        return rs;
    };
    auto copy = [&](f16 *buf, const Item &q, int k) {
        int valid = q.live ? q.rows - k * T : 0;
        valid = valid < 0 ? 0 : (valid > T ? T : valid);
        const int64_t r0 = valid > 0 ? q.t0 + (int64_t)k * T : 0;
        const int64_t bo = ((q.b * l + r0) * g + q.gi) * N;
        block_copy<P, N, HP, true>(buf, spare, x + ((q.b * l + r0) * h + q.hh0) * P, Bm + bo,
                                   Cm + bo, xs, bs, valid, wave, lane);
    };

    f32x4 accH[CPW * RT];
    // Requests the item's boundary state into accH (fp16 bits in the low
    // half of each register quad; 16 operations per lane).
    auto h_load = [&](const Item &q) {
        const int hh = q.hh0 + hs;
        const bool have = q.live && (q.c > 0 || has_init);
        const Rsrc rh = make_rsrc(Hb + ((q.b * nc + q.c) * h + hh) * NP, have ? NP * 2 : 0);
#pragma unroll
        for (int u = 0; u < CPW; ++u)
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) {
                const uint32_t off =
                    (uint32_t)((c0 + col_of<CPW>(u, li)) * N + tr * 16 + 4 * lg) * 2u;
                const u32x2 raw = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(rh, off, 0, 0));
                accH[u * RT + tr] = f32x4{as_f32(raw[0]), as_f32(raw[1]), 0.f, 0.f};
            }
    };
    auto h_convert = [&](const Item &q) {
        const int hh = q.hh0 + hs;
        const bool have = q.c > 0 || has_init;
        const float sc = have ? Hs[(q.b * h + hh) * nc + q.c] : 0.f;
#pragma unroll
        for (int t = 0; t < CPW * RT; ++t) {
            const f16x4 hv =
                __builtin_bit_cast(f16x4, u32x2{as_u32(accH[t][0]), as_u32(accH[t][1])});
            accH[t] = f32x4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]} * sc;
        }
    };

    float a2 = A[it.hh0 + hs] * kLog2e;
    float bias = dt_bias ? dt_bias[it.hh0 + hs] : 0.f;
    float Dh = D ? D[it.hh0 + hs] : 0.f;
    RowSrc rs = rsrc_of(it);

    RowIn ri;
    rows_load<SEQ>(ri, rs, 0, lane);
    copy(lds0, it, 0);
    h_load(it);
    vm_wait<0>();
    rows_prep<SEQ>(rows0[wave], ri, a2, bias, softplus, dt_min, dt_max, 0, it.rows, lane);
    h_convert(it);
    int k = 0;

    // One block of one wave; `last`: the item's last block (no carry; the
    // next item's boundary state is requested once the read-out is done).
    auto compute = [&](const f16 *buf, const Rows &rf, const Item &q, int kb, bool last,
                       const Item &nq) {
        // buffer layout as block_copy fills it: [x of each head | B | C]
        const f16 *Bs = buf + K::XE;
        const f16 *Cs = buf + K::XE + K::BE;
        const f16 *Xs = buf + hs * T * P;
        // ---- G^T tiles and the state read-out, sharing the C fragments.
        //      gt[k]: tiles (it, jt) = (0,0), (1,0), (1,1); element r of lane
        //      l: j = 16 jt + 4 lg + r, i = 16 it + li.  yh[it][u]: H^T C^T
        //      for rows 16 it.. and columns c0 + col_of(u, ..)
        f32x4 gt[3], yh[2][CPW];
#pragma unroll
        for (int e = 0; e < 3; ++e) gt[e] = zero4();
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int u = 0; u < CPW; ++u) yh[i2][u] = zero4();
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const bf16x8 c0f = rows_frag<N>(Cs, 0, 32 * m, lane);
            const bf16x8 c1f = rows_frag<N>(Cs, 16, 32 * m, lane);
            const bf16x8 b0f = rows_frag<N>(Bs, 0, 32 * m, lane);
            const bf16x8 b1f = rows_frag<N>(Bs, 16, 32 * m, lane);
            gt[0] = mma(b0f, c0f, gt[0]);
            gt[1] = mma(b0f, c1f, gt[1]);
            gt[2] = mma(b1f, c1f, gt[2]);
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const HL hf = split_acc(accH[u * RT + 2 * m], accH[u * RT + 2 * m + 1]);
                yh[0][u] = mma(hf.hi, c0f, yh[0][u]);
                yh[0][u] = mma(hf.lo, c0f, yh[0][u]);
                yh[1][u] = mma(hf.hi, c1f, yh[1][u]);
                yh[1][u] = mma(hf.lo, c1f, yh[1][u]);
            }
        }
        if (last) {
            issue_fence();
            h_load(nq);
            issue_fence();
        }

        // ---- masked, decayed scores pv[it][jt] (registers)
        const float lam = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, rf.lcs[T - 1])));
        f32x4 pv[2][2];
        float colscale[2];
        pv[0][1] = zero4();
        if (lam > -kSplit) {
            const float s15 = exp2_fast(rf.lcs[15]);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&rf.bw[4 * lg]);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&rf.bw[16 + 4 * lg]);
            const f32x2 ap = *reinterpret_cast<const f32x2 *>(&rf.a2[2 * li]);
            colscale[0] = ap[0] * s15;
            colscale[1] = ap[1] * s15;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j0 = 4 * lg + r;
                pv[0][0][r] = (j0 <= li) ? gt[0][r] * (ap[0] * b0[r]) : 0.f;
                pv[1][0][r] = gt[1][r] * (ap[1] * b0[r]);
                pv[1][1][r] = (j0 <= li) ? gt[2][r] * (ap[1] * b1[r]) : 0.f;
            }
        } else {
            const f32x2 lp = *reinterpret_cast<const f32x2 *>(&rf.l2[2 * li]);
            colscale[0] = exp2_fast(lp[0]);
            colscale[1] = exp2_fast(lp[1]);
            const f32x4 lj0 = *reinterpret_cast<const f32x4 *>(&rf.lcs[4 * lg]);
            const f32x4 lj1 = *reinterpret_cast<const f32x4 *>(&rf.lcs[16 + 4 * lg]);
            const f32x4 dj0 = *reinterpret_cast<const f32x4 *>(&rf.d[4 * lg]);
            const f32x4 dj1 = *reinterpret_cast<const f32x4 *>(&rf.d[16 + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j0 = 4 * lg + r;
                pv[0][0][r] = (j0 <= li) ? gt[0][r] * exp2_fast(lp[0] - lj0[r]) * dj0[r] : 0.f;
                pv[1][0][r] = gt[1][r] * exp2_fast(lp[1] - lj0[r]) * dj0[r];
                pv[1][1][r] = (j0 <= li) ? gt[2][r] * exp2_fast(lp[1] - lj1[r]) * dj1[r] : 0.f;
            }
        }
        if constexpr (SEQ) {
            // packed sequences: scores only between rows of one document,
            // and the state entering the block only for rows before its
            // first reset
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
        //      element r of lane l is (p = c0 + col_of(u, 4 lg + r), i = 16 it + li)
        const int r0 = kb * T;
        int valid = q.rows - r0;
        valid = valid < 0 ? 0 : (valid > T ? T : valid);
        const Rsrc ry = make_rsrc(y + ((q.b * l + q.t0 + (valid > 0 ? r0 : 0)) * h + q.hh0) * P,
                                  (int64_t)valid * xs * 2);
        bf16x8 xf[CPW];
#pragma unroll
        for (int u = 0; u < CPW; ++u) xf[u] = x_frag<CPW, P>(Xs, c0, u, lane);
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
            const int i = i2 * 16 + li;
            const HL pf = split_acc(pv[i2][0], pv[i2][1]);
            f32x4 yv[CPW];
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                f32x4 yp = mma(xf[u], pf.hi, zero4());
                yp = mma(xf[u], pf.lo, yp);
                yv[u] = colscale[i2] * yh[i2][u] + yp;
            }
            if constexpr (CPW % 2 == 0) {
                // tiles 2v, 2v + 1: 8 consecutive columns c0 + 32 v + 8 lg ..
#pragma unroll
                for (int vv = 0; vv < CPW / 2; ++vv) {
                    const f32x4 lo = yv[2 * vv], hi = yv[2 * vv + 1];
                    const uint32_t off =
                        (uint32_t)(i * xs + hs * P + c0 + 32 * vv + 8 * lg) * 2u;
                    const bf16x4 a{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3]};
                    const bf16x4 bq{(bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
                    const u32x2 ua = __builtin_bit_cast(u32x2, a),
                                ub = __builtin_bit_cast(u32x2, bq);
                    buf_store16(ry, off, u32x4{ua[0], ua[1], ub[0], ub[1]});
                }
            } else {
#pragma unroll
                for (int u = 0; u < CPW; ++u) {
                    const uint32_t off =
                        (uint32_t)(i * xs + hs * P + c0 + col_of<CPW>(u, 4 * lg)) * 2u;
                    const bf16x4 o{(bf16)yv[u][0], (bf16)yv[u][1], (bf16)yv[u][2],
                                   (bf16)yv[u][3]};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), ry, off,
                                                          0, 0);
                }
            }
        }

        // ---- carry the state to the next block of the item
        if (!last) {
            // packed sequences: nothing carried across a reset in the block
            const float decay = (SEQ && rf.seg[T - 1] >= 0) ? 0.f : exp2_fast(lam);
            HL xw[CPW];
#pragma unroll
            for (int u = 0; u < CPW; ++u) xw[u] = xw_split(xf[u], lane, rf.w);
#pragma unroll
            for (int t = 0; t < CPW * RT; ++t) accH[t] *= decay;
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) {
                const bf16x8 bt = kmajor_frag<N>(Bs, tr * 16, lane);
#pragma unroll
                for (int u = 0; u < CPW; ++u) {
                    accH[u * RT + tr] = mma(bt, xw[u].hi, accH[u * RT + tr]);
                    accH[u * RT + tr] = mma(bt, xw[u].lo, accH[u * RT + tr]);
                }
            }
        }
    };

    for (;;) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f16 *const bk = half == 0 ? lds0 : lds1;
            f16 *const bn = half == 0 ? lds1 : lds0;
            Rows &Rk = half == 0 ? rows0[wave] : rows1[wave];
            Rows &Rn = half == 0 ? rows1[wave] : rows0[wave];
            lds_barrier();
            Item nx = it;
            int kn = k + 1;
            const bool last = kn >= it.nblk;
            if (last) {
                nx = decode_item(item + G, items, nc, hpg, h, g, l, Q, HP);
                kn = 0;
            }
            const RowSrc rsn = nx.live ? rsrc_of(nx) : rs;
            RowIn rn;
            copy(bn, nx, kn);
            rows_load<SEQ>(rn, rsn, nx.live ? kn : 1 << 20, lane);
            issue_fence();
            compute(bk, Rk, it, k, last, nx);
            if (!nx.live) {
                vm_wait<0>();
                return;
            }
            // the next block's copy and rows (and with a new item its
            // boundary state) have landed; only this block's y stores may
            // still be in flight
            vm_wait<NS>();
            if (last) {
                item += G;
                it = nx;
                rs = rsn;
                a2 = A[it.hh0 + hs] * kLog2e;
                bias = dt_bias ? dt_bias[it.hh0 + hs] : 0.f;
                Dh = D ? D[it.hh0 + hs] : 0.f;
            }
            k = kn;
            rows_prep<SEQ>(Rn, rn, a2, bias, softplus, dt_min, dt_max, k, it.rows, lane);
            if (last) h_convert(it);
        }
    }
}

}  // namespace s16

// ----------------------------------------------------------------------------
template <int P, int N>
hipError_t launch_scan16(const ScanPlan &pl, const ScanArgs &a, hipStream_t s) {
    using namespace s16;
    f16 *Hb = reinterpret_cast<f16 *>(a.ws + pl.off_hb);
    f16 *St = reinterpret_cast<f16 *>(a.ws + pl.off_st);
    float *Lam = reinterpret_cast<float *>(a.ws + pl.off_lam);
    float *Smax = reinterpret_cast<float *>(a.ws + pl.off_scl);
    float *Hs = reinterpret_cast<float *>(a.ws + pl.off_hs);
    float *Imax = reinterpret_cast<float *>(a.ws + pl.off_imx);
    const bf16 *x = static_cast<const bf16 *>(a.x);
    const bf16 *dt = static_cast<const bf16 *>(a.dt);
    const bf16 *Bm = static_cast<const bf16 *>(a.B);
    const bf16 *Cm = static_cast<const bf16 *>(a.C);
    bf16 *y = static_cast<bf16 *>(a.y);
    const int h = (int)pl.h, g = (int)pl.g;
    constexpr int HPG = P >= 64 ? 128 / P : 4;
    const bool grouped = HPG > 1 && group_heads(P, h / g) == HPG;
    // the last chunk's own state only feeds the final state and the state
    // after the last chunk; chunk 0 also reports the initial state's size
    const bool keep_last = a.final_state != nullptr || a.states != nullptr;
    int64_t nc_state = keep_last ? pl.nc : pl.nc - 1;
    if (a.init && nc_state < 1) nc_state = 1;
    const bool seq = a.seq != nullptr;
    const int cus = device_cus();

    auto launch_state = [&](auto hp_c, auto seq_c) -> hipError_t {
        constexpr int HP = decltype(hp_c)::value;
        constexpr bool SQ = decltype(seq_c)::value;
        constexpr int NT = Shape<P, N, HP>::NT;
        const int64_t items = pl.b * nc_state * (h / HP);
        if (items <= 0) return hipSuccess;
        int64_t G = (int64_t)cus * resident_per_cu<&k_state16<P, N, HP, SQ>>(NT);
        G = G < items ? G : items;
        return launch_timed(&k_state16<P, N, HP, SQ>, dim3((unsigned)G), dim3(NT), s, a.ev,
                            kSlotState, x, Bm, dt, a.A, a.dt_bias, a.softplus, a.dt_min,
                            a.dt_max, a.seq, a.init, St, Smax, Lam, Imax, pl.l, h, g, pl.Q,
                            pl.nc, nc_state, items);
    };
    auto launch_out = [&](auto hp_c, auto seq_c) -> hipError_t {
        constexpr int HP = decltype(hp_c)::value;
        constexpr bool SQ = decltype(seq_c)::value;
        constexpr int NT = Shape<P, N, HP>::NT;
        const int64_t items = pl.b * pl.nc * (h / HP);
        int64_t G = (int64_t)cus * resident_per_cu<&k_out16<P, N, HP, SQ>>(NT);
        G = G < items ? G : items;
        return launch_timed(&k_out16<P, N, HP, SQ>, dim3((unsigned)G), dim3(NT), s, a.ev,
                            kSlotOut, x, Bm, Cm, dt, a.A, a.D, a.dt_bias, a.softplus, a.dt_min,
                            a.dt_max, a.seq, Hb, Hs, y, pl.l, h, g, pl.Q, pl.nc,
                            a.init != nullptr ? 1 : 0, items);
    };
    typedef std::integral_constant<int, 1> One;
    typedef std::integral_constant<int, HPG> Grp;
    typedef std::true_type Yes;
    typedef std::false_type No;

    hipError_t e = grouped ? (seq ? launch_state(Grp{}, Yes{}) : launch_state(Grp{}, No{}))
                           : (seq ? launch_state(One{}, Yes{}) : launch_state(One{}, No{}));
    if (e != hipSuccess) return e;

    const int64_t np4 = (int64_t)N * P / 4;
    const int64_t tot = pl.b * pl.h * np4;
    const unsigned scan_blocks = (unsigned)((tot + kThreads - 1) / kThreads);
    if (keep_last)
        e = launch_timed(&k_scan16<N, true>, dim3(scan_blocks), dim3(kThreads), s, a.ev,
                         kSlotScan, St, Smax, Lam, Imax, a.init, Hb, Hs, a.final_state,
                         pl.b * pl.h, h, pl.nc, N, P, a.states);
    else
        e = launch_timed(&k_scan16<N, false>, dim3(scan_blocks), dim3(kThreads), s, a.ev,
                         kSlotScan, St, Smax, Lam, Imax, a.init, Hb, Hs, (float *)nullptr,
                         pl.b * pl.h, h, pl.nc, N, P, (float *)nullptr);
    if (e != hipSuccess) return e;

    return grouped ? (seq ? launch_out(Grp{}, Yes{}) : launch_out(Grp{}, No{}))
                   : (seq ? launch_out(One{}, Yes{}) : launch_out(One{}, No{}));
}

}  // namespace ssd
