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
// removed by a select, so no inf * 0 reaches a result.  The carried state
// is held with its decay deferred (see kDefer), so most blocks only add
// their rows.
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
// Work items: (batch, chunk, HP heads of one group), one workgroup each,
// one wave per head up to head_dim 64 (two for head_dim 128).
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
// The chunk-state pass and the chunk output give one workgroup to each
// (batch, chunk, heads) item, which walks the chunk's 32-row blocks with the
// copy of the next block in flight while the current one is computed.  Both
// compute the per-row time step, cumulative decay and weights of each block
// from the raw time steps with the same code, so they agree bit for bit.
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
// The bf16 pairs (-1, 0) and (0, -1), held in registers: the compiler
// writes (-1, 0) as the inline constant -1.0, which the hardware reads as
// the fp32 value -1.0, i.e. the pair (0, -1), so the constant is hidden
// from it.
struct Neg1 {
    bf16x2 lo, hi;
};
__device__ __forceinline__ Neg1 neg1() {
    uint32_t a = 0x0000bf80u, b = 0xbf800000u;
    asm volatile("" : "+v"(a), "+v"(b));
    return Neg1{__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b)};
}
// hi = bf16(v) (nearest); v - hi is exact in fp32 and is formed with one
// bf16 dot product per value (hi times -1 in one half and 0 in the other,
// plus v), then rounded to bf16 as lo.
//
// The residuals use the dot product form whose accumulator is a separate
// operand (the builtin selects the form that overwrites its accumulator,
// which costs a register copy per value while v stays live, as the carried
// state does).  That form is written here in one assembly statement, so
// the wait states the compiler inserts for its own instructions are kept by
// hand: a dot product's result is read by another vector instruction only
// three or more instructions later (all eight products come before the
// four conversions), and the statement ends with two wait states so that a
// matrix instruction may read lo right after it.  hi is converted outside,
// so the compiler orders that first read of v (possibly a matrix result).
__device__ __forceinline__ HL split8(const float (&v)[8], const Neg1 &m) {
    HL o;
    bf16x2 h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = __builtin_convertvector((f32x2{v[2 * e], v[2 * e + 1]}), bf16x2);
        o.hi[2 * e] = h[e][0];
        o.hi[2 * e + 1] = h[e][1];
    }
    uint32_t l0, l1, l2, l3;
    float t0, t1, t2, t3, t4, t5, t6, t7;
    asm("v_dot2_f32_bf16 %4, %12, %16, %18\n\t"
        "v_dot2_f32_bf16 %5, %12, %17, %19\n\t"
        "v_dot2_f32_bf16 %6, %13, %16, %20\n\t"
        "v_dot2_f32_bf16 %7, %13, %17, %21\n\t"
        "v_dot2_f32_bf16 %8, %14, %16, %22\n\t"
        "v_dot2_f32_bf16 %9, %14, %17, %23\n\t"
        "v_dot2_f32_bf16 %10, %15, %16, %24\n\t"
        "v_dot2_f32_bf16 %11, %15, %17, %25\n\t"
        "v_cvt_pk_bf16_f32 %0, %4, %5\n\t"
        "v_cvt_pk_bf16_f32 %1, %6, %7\n\t"
        "v_cvt_pk_bf16_f32 %2, %8, %9\n\t"
        "v_cvt_pk_bf16_f32 %3, %10, %11\n\t"
        "s_nop 1"
        : "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3), "=&v"(t0), "=&v"(t1), "=&v"(t2),
          "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
        : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(m.lo), "v"(m.hi), "v"(v[0]),
          "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
    o.lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
    return o;
}
// Two accumulator tiles (contraction blocks 0..15 and 16..31 of a 32-block)
// as one operand in the k convention of ssd_device.hpp.
__device__ __forceinline__ HL split_acc(const f32x4 &t0, const f32x4 &t1, const Neg1 &m) {
    const float v[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    return split8(v, m);
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
// A value the compiler must take as changed here: the per-block LDS
// addresses derived from it are then computed afresh in every block instead
// of being kept live (or spilled) across the whole block loop.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// ------------------------------------------------------------ shapes ----
// HP heads of one group per workgroup (they share the staged B and C),
// WPH waves per head, each owning PW head_dim columns (CPW column tiles of
// 16) of its head: one wave per head up to head_dim 64 (so the per-block
// work that does not depend on the columns, the scores and the per-row
// values, is done once per head), two for head_dim 128; WH > 0 sets WPH
// (the split layouts of head_dim 64, two waves of 32 columns).
template <int P, int N, int HP, int WH = 0> struct Shape {
    static constexpr int WPH = WH > 0 ? WH : (P >= 128 ? P / 64 : 1);
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
    // y stores per lane and block (rows li and 16 + li; 8 columns a store)
    static constexpr int NS = 2 * (CPW >= 2 ? CPW / 2 : 1);
    // workgroups per compute unit the registers are budgeted for: waves
    // holding a large state (more than 64 accumulator registers) get up to
    // 256 registers (two waves per SIMD), others up to 168 (three)
    static constexpr int WPS = CPW * RT > 16 ? 2 : 3;
    static constexpr int MINB = WPS * 4 / W > 0 ? WPS * 4 / W : 1;
    static_assert(XE % 512 == 0 && BE % 512 == 0, "whole copy instructions");
    static_assert(CPW == 1 || CPW == 2 || CPW == 4, "column tiles per wave");
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

// The k-major x fragment weighted row by row (rows 4g + r and 16 + 4g + r
// of lane group g) by w, as two bf16 terms.
__device__ __forceinline__ HL xw_split(const bf16x8 &xf, int lane, const float *w,
                                       const Neg1 &m) {
    const int g = lane >> 4;
    const f32x4 wa = *reinterpret_cast<const f32x4 *>(w + 4 * g);
    const f32x4 wb = *reinterpret_cast<const f32x4 *>(w + 16 + 4 * g);
    const u32x4 xb = __builtin_bit_cast(u32x4, xf);
    const float v[8] = {bf16_lo(xb[0]) * wa[0], bf16_hi(xb[0]) * wa[1],
                        bf16_lo(xb[1]) * wa[2], bf16_hi(xb[1]) * wa[3],
                        bf16_lo(xb[2]) * wb[0], bf16_hi(xb[2]) * wb[1],
                        bf16_lo(xb[3]) * wb[2], bf16_hi(xb[3]) * wb[3]};
    return split8(v, m);
}

// State-row order.  Accumulator tile tr = 2m + h of a state (rows 16 tr..,
// element r of lane group g) holds state row
//     sigma(16 tr + 4g + r) = 32m + 8g + 4h + r,
// so that the two tiles 2m, 2m + 1 of a lane, taken as one operand (k =
// 4g + r and 16 + 4g + r of the contraction block m), meet 8 consecutive
// state rows 32m + 8g .. 32m + 8g + 7: the matching B and C fragments are
// one 16-byte LDS read each.  The B^T fragments of the carry read B's
// columns in the same order, and the stored states are written and read in
// the true order.
//
// Per-lane LDS element offsets of a wave's fragment reads inside the
// regions of a block buffer, computed once per work item.  Every fragment of
// a block is then one XOR (or add) away from them:
//   frag_rows  rows of B or C (row l & 15; k = state rows 32m + 8g ..
//              32m + 8g + 7): rows ^ 32m; rows 16..31: + 16 N
//   frag_kmaj  B^T of state-row tile 2m + h (k = the block rows 4g + r and
//              16 + 4g + r): (kmaj ^ 32m) + 4h; rows 16..31: + 16 N
//   frag_x     x of column tile u (k = the block rows): (x ^ 32 (u >> 1))
//              + 4 (u & 1), rows 16..31: + 16 P
// (the XORs only touch bits below log2 N, and a block buffer's offset is a
// multiple of N, so it can be added to the bases first).
template <int P, int N, int CPW> struct FragBase {
    int rows, kmaj, x;
    __device__ __forceinline__ void init(int c0, int lane) {

        typedef Swz<f16, N> S;
        const int g = lane >> 4, j = lane & 15;
        rows = j * N + ((g ^ S::f(j)) << 3);
        const int r = 4 * g + (j >> 2);
        kmaj = r * N + (((j & 3) ^ S::f(r)) << 3);
        if constexpr (CPW >= 2)
            x = r * P + ((((c0 >> 3) + (j & 3)) ^ xsw<P>(r)) << 3);
        else
            x = r * P + ((((c0 >> 3) + ((j >> 1) & 1)) ^ xsw<P>(r)) << 3) + 4 * (j & 1);
    }
};
// State row of element r of lane group g in accumulator tile tr.
__device__ __forceinline__ int state_row(int tr, int g) {
    return 32 * (tr >> 1) + 8 * g + 4 * (tr & 1);
}
__device__ __forceinline__ bf16x8 frag_rows(const f16 *M, int base, int m) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(M + (base ^ (32 * m))));
}
__device__ __forceinline__ f16x4 ds_tr(const f16 *p) {
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)p));
}
template <int N> __device__ __forceinline__ bf16x8 frag_kmaj(const f16 *M, int base, int tr) {
    const int o = (base ^ (32 * (tr >> 1))) + 4 * (tr & 1);
    return as_bf16x8(ds_tr(M + o), ds_tr(M + o + 16 * N));
}
template <int P> __device__ __forceinline__ bf16x8 frag_x(const f16 *Xs, int base, int u) {
    const int o = (base ^ (32 * (u >> 1))) + 4 * (u & 1);
    return as_bf16x8(ds_tr(Xs + o), ds_tr(Xs + o + 16 * P));
}

// -------------------------------------------------- per-row values ----
// Per-row values of one block of one head, kept by each wave for its own
// head in LDS (pairs (i, i + 16) interleaved where a lane reads both rows it
// owns at once).
struct alignas(16) Rows {
    float lcs[T];  // cumulative log2 decay inside the block (inclusive)
    float d[T];    // processed time step (0 past the chunk's end)
    float w[T];    // weight of row j in the carried state (see rows_prep)
    float a2[T];   // 2^(lcs_i - lcs_15), pairs (i, i + 16) at 2 (i % 16)
    float l2[T];   // lcs_i in the same pairs
    float bw[T];   // 2^(lcs_15 - lcs_j) d_j
    int seg[T];    // packed sequences: the last row <= i of the block that starts a
                   // new document, or -1
    float lam;     // the block's log2 decay (-inf across a reset)
    float dsh;     // deferred log2 decay D of the state entering the block
    float mexp;    // rebasing blocks: the carried state is first scaled by 2^mexp
    float next;    // D of the state leaving the block
    int rebase;    // the block rebases the carried state (else it defers its decay)
};
// Deferred decay.  A carried state is held as H~ = 2^D H (D >= 0, uniform
// per head), so a block whose rows leave D at most kDefer only adds its
// rows, with weights w_j = 2^(D - lcs_j) d_j <= 2^kDefer d_j, and multiplies
// nothing: its read-out scales row i by 2^(lcs_i - D), and the next block's
// D grows by -lam.  A block that would take D past kDefer (or holds a reset)
// rebases instead: H~ <- 2^(lam - D) H~ + B^T (w x) with w_j = 2^(lam - lcs_j)
// d_j, and D = 0 after it.
constexpr float kDefer = 32.f;
__device__ __forceinline__ int row_pair(int r) { return 2 * (r & 15) + (r >> 4); }


// Raw per-row inputs of one block for one head: lane l holds row l & 31
// (the two halves of a wave hold the same rows), as loaded: the values are
// first used in rows_prep, after the wait for the block's copy, so the loads
// stay in flight while the current block is computed.
struct RowIn {
    uint32_t dt;   // bf16 bits
    int cur, prv;  // packed sequences: document index of the row and of the token before
};

// Loads block k's raw rows of one head (one vector memory operation per
// lane, three with packed sequences).  dts: the head's time steps of the
// whole sequence (rows h apart); seq: the sequence's document indices; t0:
// the chunk's first token.  Rows past the sequence read as zero (rows past
// the chunk are read but not used).  rev: row t is the tensors' row
// l - 1 - t (its time step row l - 1 - t + dshift); the token before it is
// the tensors' next one.
template <bool SEQ>
__device__ __forceinline__ void rows_load(RowIn &f, const bf16 *dts, const int32_t *seq,
                                          int64_t t0, int64_t l, int h, int k, int lane, int rev,
                                          int dshift) {
    const int r = lane & 31;
    const int64_t t = t0 + (int64_t)k * T + r;
    // source rows outside [0, l) give offsets past the range (unsigned)
    const int64_t src = rev ? l - 1 - t + dshift : t;
    const Rsrc rd = make_rsrc(dts, l * h * 2);
    f.dt = __builtin_amdgcn_raw_buffer_load_b16(rd, (uint32_t)(src * h * 2), 0, 0);
    if constexpr (SEQ) {
        // the token before the chunk's first is read for every chunk but
        // the sequence's first, whose row 0 compares with itself
        const Rsrc rq = make_rsrc(seq, l * 4);
        const int64_t sc = rev ? l - 1 - t : t;
        const int64_t sp = t > 0 ? (rev ? l - t : t - 1) : sc;
        f.cur = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, (uint32_t)(sc * 4), 0, 0);
        f.prv = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, (uint32_t)(sp * 4), 0, 0);
    }
}

// softplus(z) = log(1 + e^z) from the hardware exp2 and log2 (about 1 ulp
// each): z itself above 20 (the difference is below 2.1e-9), a five-term
// series in t = e^z below t = 1/16 (relative error below 2e-7), otherwise
// ln 2 * log2(1 + t) (relative error below 1e-6).
__device__ __forceinline__ float softplus_fast(float z) {
    if (z > 20.f) return z;
    const float t = exp2_fast(z * kLog2e);
    if (t < 0.0625f)
        return t * (1.f - t * (0.5f - t * (1.f / 3.f - t * (0.25f - t * 0.2f))));
    return 0.69314718055994531f * __builtin_amdgcn_logf(1.f + t);
}

// v moved across lanes by the DPP control CTRL in the rows of ROWMASK;
// lanes whose source is outside the row, and rows outside the mask, get 0.
template <int CTRL, int ROWMASK> __device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROWMASK, 0xf, false));
}

// The block's per-row values for one head from its raw rows, written to R
// (lanes 0..31), for a state entering the block with deferred decay D.
template <bool SEQ>
__device__ __forceinline__ void rows_prep(Rows &R, const RowIn &f, float a2, float bias,
                                          int softplus, float lo, float hi, int k, int rows,
                                          float D, int lane, int adj = 0, bool first = false) {
    const int r = lane & 31;
    float d = 0.f;
    if (k * T + r < rows) {
        const float z = __builtin_bit_cast(float, f.dt << 16) + bias;
        d = softplus ? softplus_fast(z) : z;
        d = d < lo ? lo : d;
        d = d > hi ? hi : d;
    }
    float a = a2 * d;
    // adjoint rows: d sets the decay only, the weight is 1 (0 past the end),
    // and the sequence's first row takes no decay
    if (adj) {
        d = k * T + r < rows ? 1.f : 0.f;
        if (first && k == 0 && r == 0) a = 0.f;
    }
    // inclusive prefix sum over the block's 32 rows (each 32-lane half holds
    // the same rows): shifts by 1, 2, 4 and 8 lanes inside each 16-lane row
    // (sources outside the row add zero), then rows 1 and 3 add the last
    // lane of the row before them; all cross-lane moves are DPP, no LDS
    a += dpp_f<0x111, 0xf>(a);  // row_shr:1
    a += dpp_f<0x112, 0xf>(a);  // row_shr:2
    a += dpp_f<0x114, 0xf>(a);  // row_shr:4
    a += dpp_f<0x118, 0xf>(a);  // row_shr:8
    a += dpp_f<0x142, 0xa>(a);  // row_bcast:15 into rows 1 and 3
    const float last = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), T - 1));
    const float l15 = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), 15));
    float lam = last;
    int seg = -1;
    bool lazy = D - last <= kDefer;
    float w = exp2_fast((lazy ? D : last) - a) * d;
    if constexpr (SEQ) {
        // a row whose document index differs from the previous token's
        // starts from a zero state (token 0 starts from the initial state):
        // the block rebases, nothing before its last reset is carried
        const bool rst = k * T + r < rows && f.cur != f.prv;
        const uint32_t m = (uint32_t)(__ballot(rst) >> (lane & 32));
        if (m) {
            lazy = false;
            w = r < 31 - __builtin_clz(m) ? 0.f : exp2_fast(last - a) * d;
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
        if (r == 0) {
            R.lam = lam;
            R.dsh = D;
            R.mexp = lam - D;
            R.next = lazy ? D - last : 0.f;
            R.rebase = lazy ? 0 : 1;
        }
    }
}

// Power-of-two scale of an fp16 store: m (>= the largest magnitude) times
// inv lands below 2^15 (fp16's largest finite value is about 2^16); scale =
// 1 / inv.  Magnitudes below 2^-100 take the scale of 2^-100.
__device__ __forceinline__ int scale_exp(float m) {
    int ex = -100;
    if (m >= 0x1p-100f) frexpf(m, &ex);  // m = f 2^ex, f in [0.5, 1)
    return ex;
}

// How a call reads x and weighs its rows (ScanArgs): x row stride
// (elements) and heads per x slot; adj: unit row weights (adjoint scans).
struct Roles {
    int64_t xrow;
    int xdiv;
    int adj;
    // the chunk output's row dots (ScanArgs::dotv): source, its row stride,
    // heads per source slot, output
    const bf16 *dotv;
    int64_t dotrow;
    int dotdiv;
    float *dotout;
    int hbt;  // boundary states stored transposed (row-major [N][P])
    // rows in reversed order: row t of the call is row l - 1 - t of the
    // tensors (and its time step row l - 1 - t + dshift, past the end
    // reading as zero)
    int rev, dshift;
    // a call whose sequences are one computed chunk: the chunk output seeds
    // its state from init32 (fp32 [b, h, N, P], or zero) and writes the
    // state after its last row to final32 (or not), with no stored states
    const float *init32;
    float *final32;
};

// --------------------------------------------------- work items ----
// Item = (batch, chunk, HP consecutive heads of one group), heads fastest;
// one workgroup per item.  Workgroup ids go to the 8 XCDs round robin, and
// xcd_item keeps consecutive items on one XCD, so the heads of one (batch,
// chunk) meet in that XCD's L2.
struct Item {
    int64_t b, t0;  // batch row, the chunk's first token
    int c, hh0, gi, rows, nblk;
};
__device__ __forceinline__ Item decode_item(int64_t item, int nc, int hpg, int h, int g,
                                            int64_t l, int64_t Q, int HP) {
    Item it;
    const int hq = (int)(item % hpg);
    const int64_t bc = item / hpg;
    it.c = (int)(bc % nc);
    it.b = bc / nc;
    it.hh0 = hq * HP;
    it.gi = it.hh0 / (h / g);
    it.t0 = (int64_t)it.c * Q;
    const int64_t rem = l - it.t0;
    it.rows = (int)(rem < Q ? rem : Q);
    it.nblk = (it.rows + T - 1) / T;
    return it;
}

// LDS block buffer: [x of each head | B | C], B and C offset by 128 bytes
// from a bank-aligned position so that reads of B and C at the same
// in-matrix offset (which the compiler pairs into one instruction) fall in
// different banks.
template <int P, int N, int HP, int WH = 0> struct Buf {
    typedef Shape<P, N, HP, WH> K;
    static constexpr int XB = 0, BB = K::XE + 64, CB = BB + K::BE + 64;
    // buffer sizes a multiple of N elements (see FragBase)
    static constexpr int SIZE_B = (BB + K::BE + N - 1) / N * N;
    static constexpr int SIZE_BC = (CB + K::BE + N - 1) / N * N;
};

// Per-lane source offsets (bytes, inside a block) of the block copies of
// one wave: instruction j of the wave is wave instruction q = wave + j W of
// the block; x first (XI instructions), then B (BI), then C (BI, WITH_C).
// Each lane fetches the 16-byte source chunk its swizzled LDS slot holds.
template <int P, int N, int HP, bool WITH_C, int WH = 0> struct CopyPlan {
    typedef Shape<P, N, HP, WH> K;
    static constexpr int NJ = K::template per_wave<WITH_C>();
    // When the x and B blocks are whole multiples of W instructions, all W
    // instructions j W .. j W + W - 1 copy the same matrix, so which one a
    // wave's instruction j copies is known at compile time.
    static constexpr bool STATIC = K::XI % K::W == 0 && K::BI % K::W == 0;
    __device__ static __forceinline__ int klass(int j, int q) { return STATIC ? j * K::W : q; }
    uint32_t off[NJ];
    // rev: the block's rows are read in reversed order, row r of the block
    // from source row valid - 1 - r (offsets relative to the last valid row;
    // rows past it fall outside the range)
    __device__ __forceinline__ void init(int64_t xs, int64_t bs, int wave, int lane, int rev) {
        constexpr int CH = P / 8, CB = N / 8;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int q = wave + j * K::W, qc = klass(j, q);
            if (qc < K::XI) {
                const int s = q * 64 + lane;
                const int hs = s / (T * CH), rem = s % (T * CH), r = rem / CH, kk = rem % CH;
                const int64_t rs = rev ? -(int64_t)r * xs : (int64_t)r * xs;
                off[j] = (uint32_t)(rs + hs * P + ((kk ^ xsw<P>(r)) << 3)) * 2u;
            } else if (qc < K::XI + K::BI * (WITH_C ? 2 : 1)) {
                const int qb = q - K::XI;
                const int s = (qb % K::BI) * 64 + lane;
                const int r = s / CB, kk = s % CB;
                const int64_t rs = rev ? -(int64_t)r * bs : (int64_t)r * bs;
                off[j] = (uint32_t)(rs + ((kk ^ Swz<f16, N>::f(r)) << 3)) * 2u;
            } else {
                off[j] = 0u;
            }
        }
    }
    // Copies a block's valid rows of x (from the WG's first head), B and C
    // into LDS buffer buf.  x, B, C: the block's first source row (rev: its
    // lowest, the last valid row of the block).
    __device__ __forceinline__ void copy(f16 *buf, f16 *spare, const bf16 *x, const bf16 *B,
                                         const bf16 *C, int64_t xs, int64_t bs, int valid,
                                         int wave, int rev) const {
        typedef Buf<P, N, HP, WH> L;
        const RsrcW rx = make_rsrc_w(x, (int64_t)valid * xs * 2);
        const RsrcW rb = make_rsrc_w(B, (int64_t)valid * bs * 2);
        const RsrcW rc = make_rsrc_w(WITH_C ? C : B, WITH_C ? (int64_t)valid * bs * 2 : 0);
        const int vm = valid > 0 ? valid - 1 : 0;
        const uint32_t ax = rev ? (uint32_t)(vm * xs * 2) : 0u;
        const uint32_t ab = rev ? (uint32_t)(vm * bs * 2) : 0u;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int q = wave + j * K::W, qc = klass(j, q);
            if (qc < K::XI) {
                lds_dma16(rx, (lds_void *)(buf + L::XB + q * 512), off[j] + ax);
            } else if (qc < K::XI + K::BI) {
                lds_dma16(rb, (lds_void *)(buf + L::BB + (q - K::XI) * 512), off[j] + ab);
            } else if (WITH_C && qc < K::XI + 2 * K::BI) {
                lds_dma16(rc, (lds_void *)(buf + L::CB + (q - K::XI - K::BI) * 512), off[j] + ab);
            } else {
                lds_dma16(rc, (lds_void *)spare, 0u);
            }
        }
    }
};

// ----------------------------------------------------------------------------
// 1. Chunk states: one workgroup per item; its chunk from a zero state,
//        S <- 2^lam S + B^T (w x)   per block (decay deferred: S~ = 2^D S),
//    each wave holding its head_dim columns of its head's state (all
//    state_dim rows) in MFMA accumulators.  A wave of every head computes
//    that head's per-row values of the next block while the current one is
//    multiplied.  At the end the state is stored transposed
//    ([head_dim][state_dim]) as fp16 times 2^(15 - e), e the exponent of the
//    head's largest magnitude m (written as Smax), with the chunk's total
//    log2 decay (Lam); chunk-0 items also write the largest magnitude of the
//    initial state of their heads (Imax).
template <int P, int N, int HP, bool SEQ, int WH>
__global__ __launch_bounds__((Shape<P, N, HP, WH>::NT), (Shape<P, N, HP, WH>::MINB)) void k_state16(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ dt,
    const float *__restrict__ A, const float *__restrict__ dt_bias, int softplus, float dt_min,
    float dt_max, const int32_t *__restrict__ seq, const float *__restrict__ init,
    f16 *__restrict__ St, float *__restrict__ Smax, float *__restrict__ Lam,
    float *__restrict__ Imax, int64_t l, int h, int g, int64_t Q, int nc, int nc_items,
    Roles md) {
    typedef Shape<P, N, HP, WH> K;
    typedef Buf<P, N, HP, WH> L;
    constexpr int CPW = K::CPW, RT = K::RT, WPH = K::WPH;
    __shared__ __attribute__((aligned(16))) f16 lds[2 * L::SIZE_B];
    __shared__ __attribute__((aligned(16))) f16 spare[CopyPlan<P, N, HP, false, WH>::STATIC ? 8 : 512];
    __shared__ Rows rows[2][HP];
    __shared__ float wmax[K::W], wimax[K::W];

    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int hs = wave / WPH, part = wave % WPH, c0 = part * K::PW;
    const int64_t xs = md.xrow, bs = (int64_t)g * N;
    const Item it = decode_item(xcd_item(blockIdx.x, gridDim.x), nc_items, h / HP, h, g, l, Q,
                                HP);
    const int hh = it.hh0 + hs;
    // the sequence's rows of x (the WG's first head's slot), B and dt
    const bf16 *xq = x + it.b * l * xs + (int64_t)(it.hh0 / md.xdiv) * P;
    const bf16 *bq = Bm + (it.b * l * g + it.gi) * N;
    const bf16 *dts = dt + it.b * l * h + hh;
    const int32_t *sq = SEQ ? seq + it.b * l : nullptr;
    const float a2 = A[hh] * kLog2e;
    const float bias = dt_bias ? dt_bias[hh] : 0.f;

    CopyPlan<P, N, HP, false, WH> cp;
    cp.init(xs, bs, wave, lane, md.rev);
    auto copy = [&](f16 *buf, int k) {
        int valid = it.rows - k * T;
        valid = valid < 0 ? 0 : (valid > T ? T : valid);
        // the block's lowest source row
        const int64_t sr =
            valid > 0 ? (md.rev ? l - it.t0 - (int64_t)k * T - valid : it.t0 + (int64_t)k * T) : 0;
        cp.copy(buf, spare, xq + sr * xs, bq + sr * bs, nullptr, xs, bs, valid, wave, md.rev);
    };

    // the chunk's first block
    RowIn ri;
    rows_load<SEQ>(ri, dts, sq, it.t0, l, h, 0, lane, md.rev, md.dshift);
    copy(lds, 0);
    vm_wait<0>();
    if (part == 0)
        rows_prep<SEQ>(rows[0][hs], ri, a2, bias, softplus, dt_min, dt_max, 0, it.rows, 0.f,
                       lane, md.adj, it.t0 == 0);

    f32x4 acc[CPW * RT];
#pragma unroll
    for (int t = 0; t < CPW * RT; ++t) acc[t] = zero4();
    float logdec = 0.f;
    float dfin = 0.f;  // deferred decay of the state after the last block

    FragBase<P, N, CPW> fb;
    fb.init(c0, lane);

    // One block (in the buffer at element offset bo): the state decays by
    // the block's total and takes its rows.
    auto compute = [&](int bo, const Rows &R) {
        const int ln = opaque(lane);
        const int bx = opaque(fb.x + bo), bk = opaque(fb.kmaj + bo);
        const Neg1 nm = neg1();
        logdec += R.lam;
        if (R.rebase) {
            const float dec = exp2_fast(R.mexp);
#pragma unroll
            for (int t = 0; t < CPW * RT; ++t) acc[t] *= dec;
        }
        const f16 *Xs = lds + L::XB + hs * T * P;
        const f16 *Bs = lds + L::BB;
        HL xw[CPW];
#pragma unroll
        for (int u = 0; u < CPW; ++u) xw[u] = xw_split(frag_x<P>(Xs, bx, u), ln, R.w, nm);
#pragma unroll
        for (int tr = 0; tr < RT; ++tr) {
            const bf16x8 bt = frag_kmaj<N>(Bs, bk, tr);
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                acc[u * RT + tr] = mma(bt, xw[u].hi, acc[u * RT + tr]);
                acc[u * RT + tr] = mma(bt, xw[u].lo, acc[u * RT + tr]);
            }
        }
    };

    // Block k in LDS buffer k & 1.  At the top of a block the barrier tells
    // that its copy and rows have landed and that every wave is done with the
    // other buffer, into which the next block is then copied.
    for (int k = 0; k < it.nblk; ++k) {
        const int cur = k & 1;
        lds_barrier();
        const bool more = k + 1 < it.nblk;
        // every wave loads the rows (past the chunk's end they read as
        // zero), so that the loaded registers need no merge before use
        RowIn rn;
        rows_load<SEQ>(rn, dts, sq, it.t0, l, h, k + 1, lane, md.rev, md.dshift);
        if (more) copy(lds + (cur ^ 1) * L::SIZE_B, k + 1);
        issue_fence();
        compute(cur * L::SIZE_B, rows[cur][hs]);
        vm_wait<0>();
        // the head's waves take turns at the next block's rows
        if (more && part == (k + 1) % WPH)
            rows_prep<SEQ>(rows[cur ^ 1][hs], rn, a2, bias, softplus, dt_min, dt_max, k + 1,
                           it.rows, rows[cur][hs].next, lane, md.adj, it.t0 == 0);
        dfin = rows[cur][hs].next;
    }

    // ---- the chunk's state: fp16 times a power of two per head
    const bool first = init != nullptr && it.c == 0;
    {
        float m = 0.f;
#pragma unroll
        for (int t = 0; t < CPW * RT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(acc[t][e]));
        float mi = 0.f;
        if (first) {
            // the initial state's largest magnitude, for the bound on the
            // boundary states' size
            const float *src = init + (it.b * h + hh) * (int64_t)N * P;
            for (int e = (part * 64 + lane) * 4; e < N * P; e += 64 * WPH * 4) {
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
    }
    lds_barrier();
    float m = 0.f, mi = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < WPH; ++w2) {
        m = fmaxf(m, wmax[hs * WPH + w2]);
        mi = fmaxf(mi, wimax[hs * WPH + w2]);
    }
    // the held state is 2^dfin times the chunk's state
    const float undo = exp2_fast(-dfin);
    m *= undo;
    const float inv = ldexpf(1.f, 15 - scale_exp(m)) * undo;
    f16 *dst = St + (((int64_t)it.b * nc + it.c) * h + hh) * (int64_t)N * P;
#pragma unroll
    for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int tr = 0; tr < RT; ++tr) {
            const f32x4 sv = acc[u * RT + tr] * inv;
            *reinterpret_cast<f16x4 *>(dst + (c0 + col_of<CPW>(u, lane & 15)) * N +
                                       state_row(tr, lane >> 4)) =
                f16x4{(f16)sv[0], (f16)sv[1], (f16)sv[2], (f16)sv[3]};
        }
    if (part == 0 && lane == 0) {
        Smax[(it.b * h + hh) * nc + it.c] = m;
        Lam[(it.b * h + hh) * nc + it.c] = logdec;
        if (first) Imax[it.b * h + hh] = mi;
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
//    ssd_scan.hpp lays them out; chunk states are loaded GA (8 where there
//    are more than 4 chunks) to 2 GA (DEEP) chunks ahead.  A (batch, head)
//    holds a whole number of waves (n p / 4 is a multiple of 64 for every
//    supported size), so its per-chunk decays and maxima are scalar loads.
template <int N, bool ROWS, bool DEEP, int GA>
__global__ __launch_bounds__(256) void k_scan16(
    const f16 *__restrict__ St, const float *__restrict__ Smax, const float *__restrict__ Lam,
    const float *__restrict__ Imax, const float *__restrict__ init, f16 *__restrict__ Hb,
    float *__restrict__ Hs, float *__restrict__ final_state, int64_t bh, int h, int64_t nc,
    int n, int p, float *__restrict__ states) {
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
    // the wave's (batch, head), as a wave-uniform value
    const int64_t wpair = __builtin_amdgcn_readfirstlane((int)pair);
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
    const float *L = Lam + wpair * nc;
    const float *Sm = Smax + wpair * nc;
    float *hsc = Hs + pair * nc;
    const int64_t ns = (final_state || states) ? nc : nc - 1;
    const int64_t klast = ns > 0 ? ns - 1 : 0;
    // Chunk states in batches of GA; with DEEP (long sequences) two batches
    // in flight: the next batch is requested before the current one is
    // applied.
    struct Batch {
        f16x4 S[GA];
        float L[GA], M[GA];
    };
    auto fetch = [&](Batch &bt, int64_t k0) {
#pragma unroll
        for (int u = 0; u < GA; ++u) {
            // past the last chunk the pass applies, the last one is read again
            const int64_t k = k0 + u < klast ? k0 + u : klast;
            bt.S[u] = S16[k * cstride];
            bt.L[u] = L[k];
            bt.M[u] = Sm[k];
        }
    };
    auto apply = [&](const Batch &bt, int64_t k0) {
#pragma unroll
        for (int u = 0; u < GA; ++u) {
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
                const float sc = ldexpf(1.f, scale_exp(bt.M[u]) - 15);
                const f32x4 S = f32x4{(float)bt.S[u][0], (float)bt.S[u][1], (float)bt.S[u][2],
                                      (float)bt.S[u][3]} * sc;
                const float dec = exp2_fast(bt.L[u]);
                H = dec * H + S;
                M = dec * M + bt.M[u];
            }
            if (ROWS && states && c < nc)
                store_state_rows(lds, H, st, live,
                                 states + ((b * nc + c) * h + hh) * (int64_t)n * p, row0, col0, p);
        }
    };
    if constexpr (DEEP) {
        Batch b0, b1;
        fetch(b0, 0);
        for (int64_t k0 = 0; k0 < nc; k0 += 2 * GA) {
            fetch(b1, k0 + GA);
            apply(b0, k0);
            if (k0 + GA >= nc) break;
            fetch(b0, k0 + 2 * GA);
            apply(b1, k0 + GA);
        }
    } else {
        // few chunks: one batch at a time, fewer registers, more waves
        for (int64_t k0 = 0; k0 < nc; k0 += GA) {
            Batch b0;
            fetch(b0, k0);
            apply(b0, k0);
        }
    }
    if (ROWS && final_state)
        store_state_rows(lds, H, st, live, final_state + pair * (int64_t)n * p, row0, col0, p);
}

// ----------------------------------------------------------------------------
// 3. Chunk output: one workgroup per item, its chunk from its boundary
//    state.  Each wave seeds its head_dim columns of the running state H
//    (all state_dim rows, MFMA accumulators) from the stored boundary state
//    and walks the chunk's blocks; per block:
//      G^T = B C^T on the 3 causal 16 x 16 tiles, and
//      P_ij = G_ij 2^(lcs_i - lcs_j) d_j (j <= i) in registers;
//      y^T = 2^(lcs_i - D) (H~^T C^T) + x^T (P + D I)^T (the skip term on
//            the scores' diagonal; H~ = 2^D H the held state), stored
//            straight from the accumulators;
//      the carry H~ += B^T (w x), after a rebase where the block needs one
//      (except after the last block).
//    The scores and the read-out share the C fragments.  The decay factor
//    of P is taken as a_i b_j with a_i = 2^(lcs_i - lcs_15) and
//    b_j = 2^(lcs_15 - lcs_j) d_j when the block's total log2 decay is above
//    -kSplit (every factor then stays inside fp32's normal range); otherwise
//    as one exponential per element.  The first wave of every head computes
//    that head's per-row values of the next block.
constexpr float kSplit = 60.f;

template <int P, int N, int HP, bool SEQ, bool DOT, bool ONE, int WH>
__global__ __launch_bounds__((Shape<P, N, HP, WH>::NT), (Shape<P, N, HP, WH>::MINB)) void k_out16(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const bf16 *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ D,
    const float *__restrict__ dt_bias, int softplus, float dt_min, float dt_max,
    const int32_t *__restrict__ seq, const f16 *__restrict__ Hb, const float *__restrict__ Hs,
    bf16 *__restrict__ y, int64_t l, int h, int g, int64_t Q, int nc, int has_init, Roles md) {
    typedef Shape<P, N, HP, WH> K;
    typedef Buf<P, N, HP, WH> L;
    constexpr int CPW = K::CPW, RT = K::RT, WPH = K::WPH, NB = K::NB, NS = K::NS;
    __shared__ __attribute__((aligned(16))) f16 lds[2 * L::SIZE_BC];
    __shared__ __attribute__((aligned(16))) f16 spare[CopyPlan<P, N, HP, true, WH>::STATIC ? 8 : 512];
    __shared__ Rows rows[2][HP];

    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int lg = lane >> 4, li = lane & 15;
    const int hs = wave / WPH, part = wave % WPH, c0 = part * K::PW;
    const int64_t xs = md.xrow, bs = (int64_t)g * N, ys = (int64_t)h * P;
    const Item it = decode_item(xcd_item(blockIdx.x, gridDim.x), nc, h / HP, h, g, l, Q, HP);
    const int hh = it.hh0 + hs;
    // the sequence's rows of x (the WG's first head's slot), y, B, C, dt
    const bf16 *xq = x + it.b * l * xs + (int64_t)(it.hh0 / md.xdiv) * P;
    bf16 *yq = y + it.b * l * ys + (int64_t)it.hh0 * P;
    const int64_t bo = (it.b * l * g + it.gi) * N;
    const bf16 *bq = Bm + bo, *cq = Cm + bo;
    const bf16 *dts = dt + it.b * l * h + hh;
    const int32_t *sq = SEQ ? seq + it.b * l : nullptr;
    const float a2 = A[hh] * kLog2e;
    const float bias = dt_bias ? dt_bias[hh] : 0.f;
    const float Dh = D ? D[hh] : 0.f;
    // block k's lowest source row (rev: its last valid row)
    auto src_row = [&](int k, int valid) -> int64_t {
        return valid > 0 ? (md.rev ? l - it.t0 - (int64_t)k * T - valid : it.t0 + (int64_t)k * T)
                         : 0;
    };

    CopyPlan<P, N, HP, true, WH> cp;
    cp.init(xs, bs, wave, lane, md.rev);
    auto copy = [&](f16 *buf, int k) {
        int valid = it.rows - k * T;
        valid = valid < 0 ? 0 : (valid > T ? T : valid);
        const int64_t sr = src_row(k, valid);
        cp.copy(buf, spare, xq + sr * xs, bq + sr * bs, cq + sr * bs, xs, bs, valid, wave,
                md.rev);
    };

    // the chunk's first block and the wave's columns of the boundary state
    // (fp16 times the chunk's scale; zero for chunk 0 without an initial
    // state)
    RowIn ri;
    rows_load<SEQ>(ri, dts, sq, it.t0, l, h, 0, lane, md.rev, md.dshift);
    copy(lds, 0);
    f32x4 accH[CPW * RT];
    if constexpr (ONE) {
        // one chunk: the initial state itself (four rows of a column), or zero
        const Rsrc ri32 = make_rsrc(md.init32 ? md.init32 + (it.b * h + hh) * (int64_t)N * P
                                              : nullptr,
                                    md.init32 ? (int64_t)N * P * 4 : 0);
        // per-lane offset of (row 8 lg, column c0 + col_of(u, li)); the row
        // tr, e part is a uniform offset
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            const uint32_t vo = (uint32_t)(8 * lg * P + c0 + col_of<CPW>(u, li)) * 4u;
#pragma unroll
            for (int tr = 0; tr < RT; ++tr)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    accH[u * RT + tr][e] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(
                                   ri32, vo, (state_row(tr, 0) + e) * P * 4, 0));
        }
        vm_wait<0>();
    } else {
        const bool have = it.c > 0 || has_init;
        const Rsrc rh = make_rsrc(Hb + (((int64_t)it.b * nc + it.c) * h + hh) * (int64_t)N * P,
                                  have ? (int64_t)N * P * 2 : 0);
        u32x2 raw[CPW * RT];
        if (md.hbt) {
            // four consecutive state rows of one column, P elements apart
#pragma unroll
            for (int u = 0; u < CPW; ++u)
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) {
                    const uint32_t o =
                        (uint32_t)(state_row(tr, lg) * P + c0 + col_of<CPW>(u, li)) * 2u;
                    uint32_t q[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        q[e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                            rh, o + (uint32_t)(e * P * 2), 0, 0);
                    raw[u * RT + tr] = u32x2{q[0] | (q[1] << 16), q[2] | (q[3] << 16)};
                }
        } else {
#pragma unroll
            for (int u = 0; u < CPW; ++u)
#pragma unroll
                for (int tr = 0; tr < RT; ++tr)
                    raw[u * RT + tr] = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                   rh,
                                   (uint32_t)((c0 + col_of<CPW>(u, li)) * N + state_row(tr, lg)) *
                                       2u,
                                   0, 0));
        }
        const float sc = have ? Hs[((int64_t)it.b * h + hh) * nc + it.c] : 0.f;
        vm_wait<0>();
#pragma unroll
        for (int t = 0; t < CPW * RT; ++t) {
            const f16x4 hv = __builtin_bit_cast(f16x4, raw[t]);
            accH[t] = f32x4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]} * sc;
        }
    }
    // one chunk: every block carries, the last one into the final state
    if (part == 0)
        rows_prep<SEQ>(rows[0][hs], ri, a2, bias, softplus, dt_min, dt_max, 0, it.rows, 0.f,
                       lane, md.adj, it.t0 == 0);

    FragBase<P, N, CPW> fb;
    fb.init(c0, lane);
    // y offsets (bytes) of rows li and 16 + li of a block, from its first
    // row: 8 consecutive columns c0 + 32 v + 8 lg .. (column tiles 2v,
    // 2v + 1) or 4 columns c0 + 4 lg .. (one tile)
    // y rows li and 16 + li of a block (rev: offsets relative to the
    // block's last valid row, completed per block)
    const uint32_t yc = (uint32_t)(hs * P + c0 + (CPW >= 2 ? 8 : 4) * lg) * 2u;
    const uint32_t yo0 = md.rev ? yc - (uint32_t)(li * ys) * 2u : yc + (uint32_t)(li * ys) * 2u;
    const uint32_t y16 = (uint32_t)(16 * ys) * 2u;
    // DOT: every output row dotted with the matching row of md.dotv over the
    // wave's columns (the head's slot of a [b, l, slots, P] tensor), from the
    // fp32 accumulators: the block's y values are kept (ykeep) and its dot
    // rows loaded (dvv) before the next block's copies are issued, and the
    // dots are formed after the block's wait, so that no wait for them
    // holds up those copies.  Output [b, l, heads, WPH] fp32.
    constexpr int DV = CPW >= 2 ? CPW / 2 : 1;
    f32x4 ykeep[DOT ? 2 : 1][DOT ? CPW : 1];
    u32x4 dvv[DOT ? 2 : 1][DOT ? DV : 1];
    const bf16 *dbase = nullptr;
    if constexpr (DOT)
        dbase = md.dotv + it.b * l * md.dotrow + (int64_t)((it.hh0 + hs) / md.dotdiv) * P + c0;

    // One block of one wave (in the buffer at element offset bo).
    auto compute = [&](int bo, const Rows &rf, int kb, bool carry) {
        const int ln = opaque(lane), lg = ln >> 4, li = ln & 15;
        const int br = opaque(fb.rows + bo), bx = opaque(fb.x + bo), bk = opaque(fb.kmaj + bo);
        const Neg1 nm = neg1();
        const f16 *Bs = lds + L::BB;
        const f16 *Cs = lds + L::CB;
        const f16 *Xs = lds + L::XB + hs * T * P;
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
            const bf16x8 c0f = frag_rows(Cs, br, m);
            const bf16x8 c1f = frag_rows(Cs + 16 * N, br, m);
            const bf16x8 b0f = frag_rows(Bs, br, m);
            const bf16x8 b1f = frag_rows(Bs + 16 * N, br, m);
            gt[0] = mma(b0f, c0f, gt[0]);
            gt[1] = mma(b0f, c1f, gt[1]);
            gt[2] = mma(b1f, c1f, gt[2]);
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const HL hf = split_acc(accH[u * RT + 2 * m], accH[u * RT + 2 * m + 1], nm);
                yh[0][u] = mma(hf.hi, c0f, yh[0][u]);
                yh[0][u] = mma(hf.lo, c0f, yh[0][u]);
                yh[1][u] = mma(hf.hi, c1f, yh[1][u]);
                yh[1][u] = mma(hf.lo, c1f, yh[1][u]);
            }
        }

        // ---- masked, decayed scores pv[it][jt] (registers)
        const float lam = rf.lcs[T - 1];
        f32x4 pv[2][2];
        float colscale[2];
        pv[0][1] = zero4();
        if (lam > -kSplit) {
            // the read-out scale 2^(lcs_i - D) as 2^(lcs_i - lcs_15) 2^(lcs_15 - D)
            const float s15 = exp2_fast(rf.lcs[15] - rf.dsh);
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
            colscale[0] = exp2_fast(lp[0] - rf.dsh);
            colscale[1] = exp2_fast(lp[1] - rf.dsh);
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
        int valid = it.rows - r0;
        valid = valid < 0 ? 0 : (valid > T ? T : valid);
        const Rsrc ry = make_rsrc(yq + src_row(kb, valid) * ys, (int64_t)valid * ys * 2);
        const uint32_t ya = md.rev ? yo0 + (uint32_t)((valid > 0 ? valid - 1 : 0) * ys) * 2u : yo0;
        bf16x8 xf[CPW];
#pragma unroll
        for (int u = 0; u < CPW; ++u) xf[u] = frag_x<P>(Xs, bx, u);
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
            const HL pf = split_acc(pv[i2][0], pv[i2][1], nm);
            f32x4 yv[CPW];
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                f32x4 yp = mma(xf[u], pf.hi, zero4());
                yp = mma(xf[u], pf.lo, yp);
                yv[u] = colscale[i2] * yh[i2][u] + yp;
                if constexpr (DOT) ykeep[i2][u] = yv[u];
            }
            const uint32_t off = i2 == 0 ? ya : (md.rev ? ya - y16 : ya + y16);
            if constexpr (CPW >= 2) {
                // tiles 2v, 2v + 1 interleave: 8 consecutive columns
                // c0 + 32 v + 8 lg ..
#pragma unroll
                for (int v = 0; v < CPW / 2; ++v) {
                    const f32x4 &ya = yv[2 * v], &yb2 = yv[2 * v + 1];
                    const bf16x4 a{(bf16)ya[0], (bf16)ya[1], (bf16)ya[2], (bf16)ya[3]};
                    const bf16x4 bq{(bf16)yb2[0], (bf16)yb2[1], (bf16)yb2[2], (bf16)yb2[3]};
                    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, bq);
                    buf_store16(ry, off + 64u * v, u32x4{ua[0], ua[1], ub[0], ub[1]});
                }
            } else {
                const bf16x4 o{(bf16)yv[0][0], (bf16)yv[0][1], (bf16)yv[0][2], (bf16)yv[0][3]};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), ry, off, 0, 0);
            }
        }

        // ---- carry the state to the next block of the chunk
        if (carry) {
            HL xw[CPW];
#pragma unroll
            for (int u = 0; u < CPW; ++u) xw[u] = xw_split(xf[u], ln, rf.w, nm);
            // a rebasing block (packed sequences: one with a reset, which
            // carries nothing from before it) scales the held state first
            if (rf.rebase) {
                const float dec = exp2_fast(rf.mexp);
#pragma unroll
                for (int t = 0; t < CPW * RT; ++t) accH[t] *= dec;
            }
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) {
                const bf16x8 bt = frag_kmaj<N>(Bs, bk, tr);
#pragma unroll
                for (int u = 0; u < CPW; ++u) {
                    accH[u * RT + tr] = mma(bt, xw[u].hi, accH[u * RT + tr]);
                    accH[u * RT + tr] = mma(bt, xw[u].lo, accH[u * RT + tr]);
                }
            }
        }
    };

    // Block k in LDS buffer k & 1, as in k_state16; only this block's y
    // stores may still be in flight when a wave waits for the next block's
    // copy.
    for (int k = 0; k < it.nblk; ++k) {
        const int cur = k & 1;
        lds_barrier();
        const bool more = k + 1 < it.nblk;
        int dvalid = 0;
        if constexpr (DOT) {
            dvalid = it.rows - k * T;
            dvalid = dvalid > T ? T : dvalid;
            const Rsrc rd = make_rsrc(dbase + src_row(k, dvalid) * md.dotrow,
                                      (int64_t)dvalid * md.dotrow * 2);
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int v = 0; v < DV; ++v) {
                    const int64_t dr = md.rev ? dvalid - 1 - (16 * i2 + li) : 16 * i2 + li;
                    const uint32_t o =
                        (uint32_t)(dr * md.dotrow + 32 * v + (CPW >= 2 ? 8 : 4) * lg) * 2u;
                    if constexpr (CPW >= 2) {
                        dvv[i2][v] = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, o, 0, 0));
                    } else {
                        const u32x2 q = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rd, o, 0, 0));
                        dvv[i2][v] = u32x4{q[0], q[1], 0u, 0u};
                    }
                }
        }
        RowIn rn;
        rows_load<SEQ>(rn, dts, sq, it.t0, l, h, k + 1, lane, md.rev, md.dshift);
        if (more) copy(lds + (cur ^ 1) * L::SIZE_BC, k + 1);
        issue_fence();
        compute(cur * L::SIZE_BC, rows[cur][hs], k, more);
        vm_wait<NS>();
        if constexpr (DOT) {
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                float sd = 0.f;
#pragma unroll
                for (int v = 0; v < DV; ++v) {
                    const u32x4 q = dvv[i2][v];
                    if constexpr (CPW >= 2) {
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            sd += ykeep[i2][2 * v][2 * e] * bf16_lo(q[e]);
                            sd += ykeep[i2][2 * v][2 * e + 1] * bf16_hi(q[e]);
                            sd += ykeep[i2][2 * v + 1][2 * e] * bf16_lo(q[2 + e]);
                            sd += ykeep[i2][2 * v + 1][2 * e + 1] * bf16_hi(q[2 + e]);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            sd += ykeep[i2][0][2 * e] * bf16_lo(q[e]);
                            sd += ykeep[i2][0][2 * e + 1] * bf16_hi(q[e]);
                        }
                    }
                }
                // the row's four lane groups hold its other columns
                sd += __shfl_xor(sd, 16, 64);
                sd += __shfl_xor(sd, 32, 64);
                const int row = 16 * i2 + li;
                const int64_t t = it.t0 + (int64_t)k * T + row;
                if (lg == 0 && row < dvalid)
                    md.dotout[((it.b * l + (md.rev ? l - 1 - t : t)) * h + hh) * WPH + part] = sd;
            }
        }
        // the head's waves take turns at the next block's rows
        if (more && part == (k + 1) % WPH)
            rows_prep<SEQ>(rows[cur ^ 1][hs], rn, a2, bias, softplus, dt_min, dt_max, k + 1,
                           it.rows, rows[cur][hs].next, lane, md.adj, it.t0 == 0);
    }
    if (ONE && md.final32 != nullptr && it.nblk > 0) {
        // the last block's carry (after the loop, so that the loop is the
        // multi-chunk kernel's): its x fragments read again, from its buffer
        const int bo = ((it.nblk - 1) & 1) * L::SIZE_BC;
        const Rows &rf = rows[(it.nblk - 1) & 1][hs];
        {
            const int ln = opaque(lane);
            const int bx = opaque(fb.x + bo), bk = opaque(fb.kmaj + bo);
            const Neg1 nm = neg1();
            const f16 *Bs = lds + L::BB;
            const f16 *Xs = lds + L::XB + hs * T * P;
            HL xw[CPW];
#pragma unroll
            for (int u = 0; u < CPW; ++u) xw[u] = xw_split(frag_x<P>(Xs, bx, u), ln, rf.w, nm);
            if (rf.rebase) {
                const float dec = exp2_fast(rf.mexp);
#pragma unroll
                for (int t = 0; t < CPW * RT; ++t) accH[t] *= dec;
            }
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) {
                const bf16x8 bt = frag_kmaj<N>(Bs, bk, tr);
#pragma unroll
                for (int u = 0; u < CPW; ++u) {
                    accH[u * RT + tr] = mma(bt, xw[u].hi, accH[u * RT + tr]);
                    accH[u * RT + tr] = mma(bt, xw[u].lo, accH[u * RT + tr]);
                }
            }
        }
        // the held state is 2^next times the state after the last row
        const float undo = exp2_fast(-rf.next);
        const Rsrc rfin = make_rsrc(md.final32 + (it.b * h + hh) * (int64_t)N * P,
                                    (int64_t)N * P * 4);
        const int ln = opaque(lane), gq = ln >> 4, lq = ln & 15;
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            const uint32_t vo = (uint32_t)(8 * gq * P + c0 + col_of<CPW>(u, lq)) * 4u;
#pragma unroll
            for (int tr = 0; tr < RT; ++tr)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __builtin_bit_cast(uint32_t, accH[u * RT + tr][e] * undo), rfin, vo,
                        (state_row(tr, 0) + e) * P * 4, 0);
        }
    }
    // no copy may still be writing this workgroup's LDS when it exits
    vm_wait<0>();
}

}  // namespace s16

// ----------------------------------------------------------------------------
template <int P, int N>
hipError_t launch_scan16(const ScanPlan &plan, const ScanArgs &a, hipStream_t s) {
    using namespace s16;
    constexpr int HPG = P >= 128 ? 2 : 4;
    const bool grouped = bf16_item_heads(P, plan.h, plan.g) == HPG;
    // the plan the kernels run on: its chunks may join several of the
    // caller's (fewer stored states; the workspace map stays the caller's)
    ScanPlan pl = plan;
    const int m = a.interval > 0 ? a.interval
                                 : bf16_state_interval(plan, a.states != nullptr, P,
                                                       !a.dotout && !a.hb_in);
    if (m > 1) {
        pl.Q = plan.Q * m;
        pl.nc = (plan.l + pl.Q - 1) / pl.Q;
    }
    f16 *Hb = a.hb_in ? const_cast<f16 *>(static_cast<const f16 *>(a.hb_in))
                      : reinterpret_cast<f16 *>(a.ws + pl.off_hb);
    f16 *St = reinterpret_cast<f16 *>(a.ws + pl.off_st);
    float *Lam = reinterpret_cast<float *>(a.ws + pl.off_lam);
    float *Smax = reinterpret_cast<float *>(a.ws + pl.off_scl);
    float *Hs = a.hs_in ? const_cast<float *>(a.hs_in) : reinterpret_cast<float *>(a.ws + pl.off_hs);
    float *Imax = reinterpret_cast<float *>(a.ws + pl.off_imx);
    const bf16 *x = static_cast<const bf16 *>(a.x);
    const bf16 *dt = static_cast<const bf16 *>(a.dt);
    const bf16 *Bm = static_cast<const bf16 *>(a.B);
    const bf16 *Cm = static_cast<const bf16 *>(a.C);
    const int h = (int)pl.h, g = (int)pl.g;
    // sequences of one computed chunk (no per-chunk states asked): the chunk
    // output alone, from the initial state to the final one
    const bool one = pl.nc == 1 && a.states == nullptr && a.hb_in == nullptr;
    const Roles md{a.xrow ? a.xrow : (int64_t)h * P, a.xdiv, a.adj,
                   static_cast<const bf16 *>(a.dotv), a.dotrow, a.dotdiv, a.dotout, a.hbt,
                   a.rev, a.dshift, one ? a.init : nullptr, one ? a.final_state : nullptr};
    // row dots only on workgroups of one head (the gradient pass's
    // transposed scans)
    if (a.dotout && grouped) return hipErrorInvalidValue;
    // the last chunk's own state only feeds the final state and the state
    // after the last chunk; chunk 0 also reports the initial state's size
    const bool keep_last = a.final_state != nullptr || a.states != nullptr;
    int64_t nc_state = keep_last ? pl.nc : pl.nc - 1;
    if (a.init && nc_state < 1) nc_state = 1;
    const bool seq = a.seq != nullptr;
    // Workgroup layout: 0 one head, 1 a group's HPG heads (one wave per head
    // up to head_dim 64), 2 HPG / 2 heads, 3 one head, both with two waves per
    // head_dim 64 head (32 columns each).  A wave of a split head holds half
    // the state (64 accumulator registers, three waves per SIMD) and repeats
    // the head's scores and per-row values.  Grouped calls split where the
    // split grid fits the chip at once (three workgroups per compute unit):
    // there the grouped grid would leave compute units with one workgroup
    // beside others with two.  Calls that are not grouped always split: one
    // head of one wave holds the B and C blocks for itself, and LDS then
    // allows only three such waves per compute unit.  The row dots of the
    // gradient pass's transposed scans keep one wave per head.
    int lay = grouped ? 1 : 0;
    if (P == 64 && !a.dotout) {
        if (!grouped)
            lay = (h / g) % 2 == 0 ? 2 : 3;
        else if (2 * pl.b * pl.nc * (h / HPG) <= 3 * (int64_t)device_cus())
            lay = 2;
    }

    typedef std::integral_constant<int, 1> One;
    typedef std::integral_constant<int, HPG> Grp;
    typedef std::true_type Yes;
    typedef std::false_type No;

    auto launch_state = [&](auto hp_c, auto wh_c, auto seq_c) -> hipError_t {
        constexpr int HP = decltype(hp_c)::value, WH = decltype(wh_c)::value;
        constexpr bool SQ = decltype(seq_c)::value;
        constexpr int NT = Shape<P, N, HP, WH>::NT;
        const int64_t items = pl.b * nc_state * (h / HP);
        if (items <= 0) return hipSuccess;
        return launch_timed(&k_state16<P, N, HP, SQ, WH>, dim3((unsigned)items), dim3(NT), s,
                            a.ev, kSlotState, x, Bm, dt, a.A, a.dt_bias, a.softplus, a.dt_min,
                            a.dt_max, a.seq, a.init, St, Smax, Lam, Imax, pl.l, h, g, pl.Q,
                            (int)pl.nc, (int)nc_state, md);
    };
    auto launch_out = [&](auto hp_c, auto wh_c, auto seq_c) -> hipError_t {
        constexpr int HP = decltype(hp_c)::value, WH = decltype(wh_c)::value;
        constexpr bool SQ = decltype(seq_c)::value;
        constexpr int NT = Shape<P, N, HP, WH>::NT;
        const int64_t items = pl.b * pl.nc * (h / HP);
        if (items <= 0) return hipSuccess;
        if constexpr (HP == 1 && WH == 0) {
            if (a.dotout && one)
                return launch_timed(&k_out16<P, N, 1, SQ, true, true, 0>, dim3((unsigned)items),
                                    dim3(NT), s, a.ev, kSlotOut, x, Bm, Cm, dt, a.A, a.D,
                                    a.dt_bias, a.softplus, a.dt_min, a.dt_max, a.seq, Hb, Hs,
                                    static_cast<bf16 *>(a.y), pl.l, h, g, pl.Q, (int)pl.nc,
                                    0, md);
            if (a.dotout)
                return launch_timed(&k_out16<P, N, 1, SQ, true, false, 0>, dim3((unsigned)items),
                                    dim3(NT), s, a.ev, kSlotOut, x, Bm, Cm, dt, a.A, a.D,
                                    a.dt_bias, a.softplus, a.dt_min, a.dt_max, a.seq, Hb, Hs,
                                    static_cast<bf16 *>(a.y), pl.l, h, g, pl.Q, (int)pl.nc,
                                    a.init != nullptr ? 1 : 0, md);
        }
        if (one)
            return launch_timed(&k_out16<P, N, HP, SQ, false, true, WH>, dim3((unsigned)items),
                                dim3(NT), s, a.ev, kSlotOut, x, Bm, Cm, dt, a.A, a.D,
                                a.dt_bias, a.softplus, a.dt_min, a.dt_max, a.seq, Hb, Hs,
                                static_cast<bf16 *>(a.y), pl.l, h, g, pl.Q, (int)pl.nc, 0, md);
        return launch_timed(&k_out16<P, N, HP, SQ, false, false, WH>, dim3((unsigned)items),
                            dim3(NT), s, a.ev, kSlotOut, x, Bm, Cm, dt, a.A, a.D, a.dt_bias,
                            a.softplus, a.dt_min, a.dt_max, a.seq, Hb, Hs,
                            static_cast<bf16 *>(a.y), pl.l, h, g, pl.Q, (int)pl.nc,
                            a.init != nullptr ? 1 : 0, md);
    };
    // runs a launcher in the call's layout: one head per workgroup, a group's
    // HPG heads, or (split) half as many heads with two waves per head
    auto dispatch = [&](auto launch) -> hipError_t {
        typedef std::integral_constant<int, 0> W0;
        if constexpr (P == 64) {
            typedef std::integral_constant<int, HPG / 2> Half;
            typedef std::integral_constant<int, 2> W2;
            if (lay == 2) return seq ? launch(Half{}, W2{}, Yes{}) : launch(Half{}, W2{}, No{});
            if (lay == 3) return seq ? launch(One{}, W2{}, Yes{}) : launch(One{}, W2{}, No{});
        }
        if (lay == 1) return seq ? launch(Grp{}, W0{}, Yes{}) : launch(Grp{}, W0{}, No{});
        return seq ? launch(One{}, W0{}, Yes{}) : launch(One{}, W0{}, No{});
    };

    // boundary states given (hb_in), or one chunk: the chunk output alone
    if (!a.hb_in && !one) {
        hipError_t e = dispatch(launch_state);
        if (e != hipSuccess) return e;

        const int64_t np4 = (int64_t)N * P / 4;
        const int64_t tot = pl.b * pl.h * np4;
        const unsigned scan_blocks = (unsigned)((tot + kThreads - 1) / kThreads);
        // chunk states requested 8 ahead, two batches in flight where there
        // are many chunks, smaller batches for 4 chunks or fewer
        auto launch_scan = [&](auto rows_c, auto deep_c, auto ga_c) -> hipError_t {
            constexpr bool RW = decltype(rows_c)::value, DP = decltype(deep_c)::value;
            constexpr int GA = decltype(ga_c)::value;
            return launch_timed(&k_scan16<N, RW, DP, GA>, dim3(scan_blocks), dim3(kThreads), s,
                                a.ev, kSlotScan, St, Smax, Lam, Imax, a.init, Hb, Hs,
                                RW ? a.final_state : (float *)nullptr, pl.b * pl.h, h, pl.nc, N, P,
                                RW ? a.states : (float *)nullptr);
        };
        auto launch_rows = [&](auto rows_c) -> hipError_t {
            typedef std::integral_constant<int, 8> G8;
            typedef std::integral_constant<int, 4> G4;
            if (pl.nc >= 64) return launch_scan(rows_c, Yes{}, G8{});
            if (pl.nc > 4) return launch_scan(rows_c, No{}, G8{});
            if (pl.nc > 1) return launch_scan(rows_c, No{}, G4{});
            return launch_scan(rows_c, No{}, One{});
        };
        e = keep_last ? launch_rows(Yes{}) : launch_rows(No{});
        if (e != hipSuccess) return e;
    }

    return dispatch(launch_out);
}

}  // namespace ssd
