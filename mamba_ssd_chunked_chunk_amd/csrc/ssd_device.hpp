// Device-side building blocks shared by the SSD scan kernels (gfx950).
//
// Matrix products run on the CDNA matrix cores through 16x16 MFMA tiles with
// fp32 accumulation: v_mfma_f32_16x16x32_f16 on the bf16 path and
// v_mfma_f32_16x16x4_f32 on the fp32 path.  On the bf16 path the operands
// are fp16: the bf16 inputs (x, B, C) convert to fp16 exactly while they lie
// in fp16's normal range, and the operands derived inside the scan (masked
// scores, decay-weighted x, the carried state) keep 11 significant bits
// instead of bf16's 8.
//
// Fragment / accumulator lane layout (wave64), with g = lane >> 4:
//   row-major A fragment (rows i0..i0+15, contraction block k0): lane l holds
//     row i0 + (l & 15), k = k0 + KPL * g + e, e < KPL;
//   row-major B fragment (columns j0..j0+15): column j0 + (l & 15), same k;
//   accumulator: element r of lane l is (i0 + 4 g + r, j0 + (l & 15)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;      // waves per workgroup of the scan kernels
constexpr int kThreads = 256;  // threads per workgroup

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }

// 2^x on the transcendental unit (v_exp_f32); 2^(-large) -> 0, never NaN
// for finite x.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Processed time step of one token: clamp(softplus(dt + bias)).  For
// z > 20 softplus(z) = z to within 2.1e-9.
__device__ __forceinline__ float time_step(float raw, float bias, int use_softplus,
                                           float lo, float hi) {
    float z = raw + bias;
    float d = use_softplus ? (z > 20.f ? z : log1pf(expf(z))) : z;
    d = d < lo ? lo : d;
    d = d > hi ? hi : d;
    return d;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Four consecutive io elements as fp32, and back (bf16 rounded to nearest even).
template <typename IO> __device__ __forceinline__ f32x4 ld4(const IO *p);
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <> __device__ __forceinline__ f32x4 ld4<bf16>(const bf16 *p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <typename IO> __device__ __forceinline__ void st4(IO *p, f32x4 v);
template <> __device__ __forceinline__ void st4<float>(float *p, f32x4 v) {
    *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ __forceinline__ void st4<bf16>(bf16 *p, f32x4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4 *>(p) = o;
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: values derived from it (head slot, column offset, buffer resources)
// then stay in scalar registers instead of being treated as per-lane.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads, so a register prefetch issued before it stays in
// flight across the barrier.  Global memory written before it is not made
// visible to other waves (no kernel here relies on that).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------------- operands ----
template <typename IO> struct Op { typedef float type; };
template <> struct Op<bf16> { typedef f16 type; };

template <typename OP> struct Mfma;
template <> struct Mfma<f16> {
    static constexpr int K = 32;   // contraction length of one instruction
    static constexpr int KPL = 8;  // contraction elements per lane
    static constexpr int PAD = 8;  // row-major LDS row padding (16 bytes)
    typedef f16x8 frag;
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int K = 4;
    static constexpr int KPL = 1;
    static constexpr int PAD = 4;
    typedef float frag;
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// Operands stored k-major in LDS (M[k][col], col contiguous) are read with
// the gfx950 transposing LDS load ds_read_b64_tr_b16: inside each group of
// 16 lanes, lane 4r + c supplies the address of elements 4c..4c+3 of row r
// of a 4 x 16 tile, and lane i receives column i of the tile's 4 rows.
// lds_tr4 returns, for lane l (group g), M[k0 + 4g + r][c0 + (l & 15)],
// r = 0..3.
typedef __fp16 fp16x4_raw __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_raw lds_fp16x4;
__device__ __forceinline__ f16x4 lds_tr4(const f16 *M, int ld, int k0, int c0, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const f16 *p = M + (k0 + 4 * g + (j >> 2)) * ld + c0 + 4 * (j & 3);
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)p));
}

// Contraction-order convention for k-major operands.  Within a block of 32
// contraction indices starting at kb, lane group g of an fp16 fragment
// carries k = kb + 4g + r (elements 0..3) and kb + 16 + 4g + r (elements
// 4..7); an fp32 MFMA step q (0..7) carries k = kb + 16 (q >> 2) + 4g + (q & 3).
// Both operands of a product use the same convention, so the sum is the same
// as in natural order.  The accumulator layout of 16 x 16 tiles (lane l holds
// rows 4g + r of column l & 15) produces values in exactly this order, so a
// product's result can feed the next product straight from registers.
__device__ __forceinline__ f16x8 frag_kmajor(const f16 *M, int ld, int kb, int, int c0,
                                             int lane) {
    const f16x4 a = lds_tr4(M, ld, kb, c0, lane);
    const f16x4 b = lds_tr4(M, ld, kb + 16, c0, lane);
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ float frag_kmajor(const float *M, int ld, int kb, int q, int c0,
                                             int lane) {
    return M[(kb + 16 * (q >> 2) + 4 * (lane >> 4) + (q & 3)) * ld + c0 + (lane & 15)];
}

// Two fp32 values -> packed fp16 pair, rounded toward zero (one instruction;
// error below 2^-11 relative).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x2 pk2(float a, float b) {
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ void pack2(float a, float b, f16 &lo, f16 &hi) {
    const f16x2 pk = pk2(a, b);
    lo = pk[0];
    hi = pk[1];
}

// An operand fragment made from two accumulator tiles (contraction blocks
// jt = 0, 1 of a 32-block) in the k-major convention above.
template <typename OP>
__device__ __forceinline__ typename Mfma<OP>::frag frag_from_acc(const f32x4 &t0,
                                                                 const f32x4 &t1, int q);
template <>
__device__ __forceinline__ f16x8 frag_from_acc<f16>(const f32x4 &t0, const f32x4 &t1, int) {
    const f16x2 a = pk2(t0[0], t0[1]), b = pk2(t0[2], t0[3]);
    const f16x2 c = pk2(t1[0], t1[1]), d = pk2(t1[2], t1[3]);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
template <>
__device__ __forceinline__ float frag_from_acc<float>(const f32x4 &t0, const f32x4 &t1, int q) {
    return (q >> 2) ? t1[q & 3] : t0[q & 3];
}

// ------------------------------------------------- swizzled LDS matrices ----
// An LDS matrix M[row][col] with NCOL columns and no row padding, whose
// 16-byte chunks are stored at chunk index (col / EPC) ^ f(row).  f maps
// rows 0..15 one-to-one onto chunk offsets, and rows 0..7 (and 8..15) onto
// distinct chunk pairs {2k, 2k + 1}; for NCOL = 128 fp16 this makes the
// row-major 16-byte fragment reads (16 rows, one chunk each), the transposing
// 8-byte reads (8 rows, two chunks each) and the row-piece stores all free of
// bank conflicts.
template <typename T, int NCOL> struct Swz {
    static constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
    static constexpr int CH = NCOL / EPC;            // chunks per row (a power of 2)
    __device__ static __forceinline__ int f(int r) {
        return ((((r & 7) << 1) | ((r >> 3) & 1))) & (CH - 1);
    }
    __device__ static __forceinline__ int at(int r, int c) {
        return r * NCOL + (((c / EPC) ^ f(r)) * EPC) + (c % EPC);
    }
};

// Row-major rows M[row][k] read in the k-major contraction convention from a
// swizzled matrix: lane l gets row row0 + (l & 15) at k = kb + 4g + r and
// kb + 16 + 4g + r (fp16), or at k = kb + 16 (q >> 2) + 4g + (q & 3) for fp32
// step q.  Pairs with a k-major or accumulator-made partner operand.
template <typename OP, int NCOL>
__device__ __forceinline__ typename Mfma<OP>::frag swz_rows_kconv(const OP *M, int row0, int kb,
                                                                  int q, int lane) {
    typedef Swz<OP, NCOL> S;
    const int r = row0 + (lane & 15), g = lane >> 4;
    if constexpr (sizeof(OP) == 2) {
        const f16x4 a = *reinterpret_cast<const f16x4 *>(M + S::at(r, kb + 4 * g));
        const f16x4 b = *reinterpret_cast<const f16x4 *>(M + S::at(r, kb + 16 + 4 * g));
        return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        return M[S::at(r, kb + 16 * (q >> 2) + 4 * g + (q & 3))];
    }
}

// k-major fragment (as frag_kmajor: rows = contraction index) of a swizzled
// matrix, through the transposing LDS read for fp16.
template <typename OP, int NCOL>
__device__ __forceinline__ typename Mfma<OP>::frag swz_kmajor(const OP *M, int kb, int q, int c0,
                                                              int lane) {
    typedef Swz<OP, NCOL> S;
    const int g = lane >> 4, j = lane & 15;
    if constexpr (sizeof(OP) == 2) {
        const f16 *pa = M + S::at(kb + 4 * g + (j >> 2), c0 + 4 * (j & 3));
        const f16 *pb = M + S::at(kb + 16 + 4 * g + (j >> 2), c0 + 4 * (j & 3));
        const f16x4 a = __builtin_bit_cast(
            f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pa));
        const f16x4 b = __builtin_bit_cast(
            f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pb));
        return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        return M[S::at(kb + 16 * (q >> 2) + 4 * g + (q & 3), c0 + j)];
    }
}

// A row piece of 8 elements stored into a swizzled matrix.
template <typename T, int NCOL, typename V>
__device__ __forceinline__ void swz_store8(T *M, int r, int c0, const V &v) {
    typedef Swz<T, NCOL> S;
    static_assert(sizeof(V) == 8 * sizeof(T), "row piece of 8 elements");
    constexpr int NV = sizeof(V) / 16;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(&v);
#pragma unroll
    for (int i = 0; i < NV; ++i)
        *reinterpret_cast<u32x4 *>(M + S::at(r, c0 + i * S::EPC)) = src[i];
}

// Paired column order for fp16 matrices contracted over their columns in the
// k convention above: inside every 32 columns, column n = 32m + 16h + 4g + r
// is kept at 32m + 8g + 4h + r, so the two 4-element halves of a fragment
// (k = kb + 4g + r and kb + 16 + 4g + r) form one 16-byte chunk, and a
// transposing read's 4 consecutive columns stay 4 consecutive elements.
__device__ __forceinline__ int pair_col(int n) {
    return (n & ~31) | (((n >> 2) & 3) << 3) | (((n >> 4) & 1) << 2) | (n & 3);
}

// Row piece of 8 consecutive columns c0 .. c0 + 7 (c0 % 8 == 0) stored into a
// swizzled matrix in paired order: two 8-byte halves.
template <int NCOL, typename V>
__device__ __forceinline__ void swzp_store8(f16 *M, int r, int c0, const V &v) {
    typedef Swz<f16, NCOL> S;
    static_assert(sizeof(V) == 16, "row piece of 8 fp16 elements");
    const u32x4 w = __builtin_bit_cast(u32x4, v);
    *reinterpret_cast<u32x2 *>(M + S::at(r, pair_col(c0))) = u32x2{w[0], w[1]};
    *reinterpret_cast<u32x2 *>(M + S::at(r, pair_col(c0 + 4))) = u32x2{w[2], w[3]};
}

// Row-major rows in the k convention from a swizzled paired matrix: one
// 16-byte read per lane.
template <int NCOL>
__device__ __forceinline__ f16x8 swzp_rows_kconv(const f16 *M, int row0, int kb, int lane) {
    typedef Swz<f16, NCOL> S;
    return *reinterpret_cast<const f16x8 *>(M + S::at(row0 + (lane & 15), kb + 8 * (lane >> 4)));
}

// k-major fragment (rows = contraction index, as frag_kmajor) of a swizzled
// paired matrix, columns c0 .. c0 + 15 in logical order.
template <int NCOL>
__device__ __forceinline__ f16x8 swzp_kmajor(const f16 *M, int kb, int c0, int lane) {
    typedef Swz<f16, NCOL> S;
    const int g = lane >> 4, j = lane & 15;
    const int pc = pair_col(c0 + 4 * (j & 3));
    const f16 *pa = M + S::at(kb + 4 * g + (j >> 2), pc);
    const f16 *pb = M + S::at(kb + 16 + 4 * g + (j >> 2), pc);
    const f16x4 a =
        __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pa));
    const f16x4 b =
        __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)pb));
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---------------------------------------------------------- row pieces ----
// 8 consecutive elements of one row, moved with vector loads and stores.
template <typename T> struct alignas(16) Row8v { T e[8]; };

template <typename T> __device__ __forceinline__ void st_row8(T *dst, const Row8v<T> &v) {
    *reinterpret_cast<Row8v<T> *>(dst) = v;
}

// ------------------------------------------------------ buffer access ----
// Raw buffer resources: loads whose offset lies at or beyond the resource's
// byte size return zeros and such stores are dropped, so rows past the end of
// a chunk or of the sequence need no masks.  Offsets are 32-bit; every
// resource here spans at most a few rows of one tensor.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (CDNA)

// Every resource here is wave-uniform by construction; the base and size are
// passed through readfirstlane so that the compiler keeps the descriptor in
// scalar registers (a descriptor it believes per-lane costs a loop per load).
__device__ __forceinline__ Rsrc make_rsrc(const void *base, int64_t bytes) {
    const int64_t c = bytes < 0 ? 0 : (bytes > 0xffffffffLL ? 0xffffffffLL : bytes);
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)(uint32_t)c);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, kRsrcWord3);
}
// One 16-byte copy per lane from a buffer resource straight into LDS: the
// wave writes 64 consecutive 16-byte slots starting at dst (lane i at
// dst + 16 i), whatever offset each lane reads; offsets past the resource
// write zeros.  The builtin exists only for the device: in the host pass
// of the compiler it would mark every template that calls it as invalid
// (the host never runs this code), so the body is compiled there as empty.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void lds_copy16(Rsrc r, lds_void *dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
#else
    (void)r, (void)dst, (void)voff;
#endif
}
// The same 16-byte copy into LDS written out as machine code, with the
// buffer descriptor as four plain words.  The compiler does not see that it
// writes LDS or that it counts in vmcnt, so it adds no wait of its own before
// later LDS reads (with the builtin it waits for every copy in flight before
// each transposing LDS read, whatever buffer the read uses): the caller
// orders the copies with vm_wait and lds_barrier.  It has no output
// register; M0 (the LDS address) is set in the same statement, with the one
// wait state the hardware needs between that write and the copy.  Waits the
// compiler adds for its own loads count only its own operations and so stay
// correct (completion is in issue order).
typedef uint32_t RsrcW __attribute__((ext_vector_type(4)));
__device__ __forceinline__ RsrcW make_rsrc_w(const void *base, int64_t bytes) {
    const int64_t c = bytes < 0 ? 0 : (bytes > 0xffffffffLL ? 0xffffffffLL : bytes);
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return RsrcW{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu,
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)c), (uint32_t)kRsrcWord3};
}
__device__ __forceinline__ void lds_dma16(RsrcW r, lds_void *dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff),
                 "s"(r), "s"(a)
                 : "memory", "m0");
#else
    (void)r, (void)dst, (void)voff;
#endif
}
template <typename T> __device__ __forceinline__ Row8v<T> buf_row8(Rsrc r, uint32_t off) {
    constexpr int NV = sizeof(Row8v<T>) / 16;
    u32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
    Row8v<T> o;
    __builtin_memcpy(&o, v, sizeof(o));
    return o;
}
__device__ __forceinline__ float buf_f32(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store16(Rsrc r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// Issue priority of this wave (0..3, uniform).  Workgroups that share a
// compute unit advance at different rates under the default oldest-first
// issue order; raising the priority of waves that are behind in their walk
// keeps them together, so the unit does not idle at the end.
__device__ __forceinline__ void wave_priority(int level) {
    if (level >= 3)
        __builtin_amdgcn_s_setprio(3);
    else if (level == 2)
        __builtin_amdgcn_s_setprio(2);
    else if (level == 1)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}
// Priority for a wave at block k of nblk: 3 at the start, 0 in the last quarter.
__device__ __forceinline__ int progress_priority(int k, int nblk) {
    return 3 - (4 * k) / (nblk > 0 ? nblk : 1);
}

// ------------------------------------------------ memory ordering ----
// Keeps the memory operations before and after it in program order, so that
// the counts given to vm_wait match the order of issue.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Wait until at most N vector memory operations of this wave are in flight
// (they complete in issue order).
template <int N> __device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ------------------------------------------------- state tiles ----
// The state scan's threads cover each (batch, head) state in tiles of R
// state rows by Cc head_dim columns (R = min(state_dim, 64), R Cc = 1024 or
// all of a small state); a thread holds 4 consecutive state rows of one
// column, the tile's threads running down the rows first.  Chunk states and
// boundary states ([head_dim][state_dim]) are then read and written in runs
// of R elements, and a tile's rows of the [state_dim][head_dim] outputs in
// runs of Cc.
struct ScanTile {
    int R, Cc, TT;  // rows, columns, threads of a tile
    __device__ ScanTile(int n, int p) {
        R = n < 64 ? n : 64;
        Cc = p < 1024 / R ? p : 1024 / R;
        TT = R * Cc / 4;
    }
};

// Stores a tile of the state ([state_dim][head_dim] order, 16 bytes per lane
// along the rows) through LDS: thread t of the tile passes its 4 elements v
// and the tile's output `out` (rows row0.., columns col0..).  Every thread of
// the workgroup takes part (two barriers, which wait for LDS only: the global
// stores before them stay in flight); `live` false stores nothing.
__device__ __forceinline__ void store_state_rows(float *lds, const f32x4 &v, const ScanTile &st,
                                                 bool live, float *out, int row0, int col0,
                                                 int p) {
    const int tid = threadIdx.x, tw = tid / st.TT, loc = tid % st.TT;
    lds_barrier();  // earlier reads of the tile are done
    *reinterpret_cast<f32x4 *>(lds + 4 * tid) = v;
    lds_barrier();
    const int v0 = 4 * loc, row = v0 / st.Cc, col = v0 % st.Cc;
    const float *t = lds + tw * st.TT * 4;
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = t[(col + i) * st.R + row];
    if (live) *reinterpret_cast<f32x4 *>(out + (int64_t)(row0 + row) * p + col0 + col) = o;
}

// ----------------------------------------------- workgroup -> work item ----
// Workgroups are handed to the 8 XCDs round-robin by id (id % 8).  Work items
// that share data (the heads of one group, the slices of one state) are
// given consecutive indices, and this map sends consecutive indices to the
// same XCD so that they meet in that XCD's L2.
__device__ __forceinline__ int64_t xcd_item(int64_t bid, int64_t nblocks) {
    const int64_t q = nblocks >> 3, r = nblocks & 7;
    const int64_t x = bid & 7, k = bid >> 3;
    return x * q + (x < r ? x : r) + k;
}

}  // namespace ssd
