// Device-side building blocks shared by the SSD scan kernels (gfx950).
//
// Matrix products run on the CDNA matrix cores through 16x16 MFMA tiles:
// v_mfma_f32_16x16x32_bf16 for bf16 operands and v_mfma_f32_16x16x4_f32 for
// fp32 operands, both accumulating in fp32.  Operand tiles are staged in LDS
// with the contraction index contiguous, so each lane reads its fragment
// with one vector load.  Fragment / accumulator lane layout (wave64):
//   A fragment of rows i0..i0+15, k block k0: lane l holds row i0 + (l & 15),
//     k = k0 + KPL * (l >> 4) + e, e < KPL;
//   B fragment of columns j0..j0+15: lane l holds column j0 + (l & 15) with
//     the same k indices;
//   accumulator: element r of lane l is (i0 + 4 * (l >> 4) + r, j0 + (l & 15)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;      // waves per workgroup of the scan kernels
constexpr int kThreads = 256;  // threads per workgroup

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// fp32 -> bf16 round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

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

// ---------------------------------------------------------------- MFMA ----
template <typename OP> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int K = 32;   // contraction length of one instruction
    static constexpr int KPL = 8;  // contraction elements per lane
    static constexpr int PAD = 8;  // LDS row padding (elements): 16 bytes
    typedef bf16x8 frag;
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// Fragment of an LDS matrix M[row][k] (k contiguous, row stride ld): lane l
// reads row `row0 + (l & 15)` at k = k0 + KPL * (l >> 4).
template <typename OP>
__device__ __forceinline__ typename Mfma<OP>::frag
lds_frag(const OP *M, int ld, int row0, int k0, int lane) {
    const OP *p = M + (row0 + (lane & 15)) * ld + k0 + Mfma<OP>::KPL * (lane >> 4);
    return *reinterpret_cast<const typename Mfma<OP>::frag *>(p);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------- 8x8 staging ------
// A thread moves one 8 x 8 block of a row-major global matrix (8 rows of 8
// consecutive elements) into LDS, either in the same orientation or
// transposed (so that the former row index becomes contiguous).

template <typename IO> struct Row8;
template <> struct Row8<bf16> {
    typedef bf16x8 vec;  // 16 bytes
};
template <> struct Row8<float> {
    struct vec { f32x4 lo, hi; };  // 32 bytes
};

template <typename IO>
__device__ __forceinline__ typename Row8<IO>::vec load_row8(const IO *p) {
    return *reinterpret_cast<const typename Row8<IO>::vec *>(p);
}
template <typename IO> __device__ __forceinline__ typename Row8<IO>::vec zero_row8() {
    typename Row8<IO>::vec v;
    __builtin_memset(&v, 0, sizeof(v));
    return v;
}

__device__ __forceinline__ float row8_get(const Row8<bf16>::vec &v, int e) { return (float)v[e]; }
__device__ __forceinline__ float row8_get(const Row8<float>::vec &v, int e) {
    return e < 4 ? v.lo[e] : v.hi[e - 4];
}

// Store 8 values (fp32 in registers) to LDS as OP, contiguous.
template <typename OP> __device__ __forceinline__ void lds_store8(OP *dst, const float *v);
template <> __device__ __forceinline__ void lds_store8<bf16>(bf16 *dst, const float *v) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8 *>(dst) = o;
}
template <> __device__ __forceinline__ void lds_store8<float>(float *dst, const float *v) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Store 4 fp32 values to LDS as OP, contiguous (8 or 16 bytes).
template <typename OP> __device__ __forceinline__ void lds_store4(OP *dst, f32x4 v);
template <> __device__ __forceinline__ void lds_store4<bf16>(bf16 *dst, f32x4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4 *>(dst) = o;
}
template <> __device__ __forceinline__ void lds_store4<float>(float *dst, f32x4 v) {
    *reinterpret_cast<f32x4 *>(dst) = v;
}

// Load 4 contiguous OP values from LDS as fp32.
template <typename OP> __device__ __forceinline__ f32x4 lds_load4(const OP *src);
template <> __device__ __forceinline__ f32x4 lds_load4<bf16>(const bf16 *src) {
    bf16x4 v = *reinterpret_cast<const bf16x4 *>(src);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <> __device__ __forceinline__ f32x4 lds_load4<float>(const float *src) {
    return *reinterpret_cast<const f32x4 *>(src);
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
