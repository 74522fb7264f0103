// The two steps around the scan in a Mamba-2 mixer, each one pass over HBM
// (the transformers issue page on the layer's two paths: a short causal
// conv1d, then the chunk scan; nnterp guide: the heads' y is read before the
// gated norm and the output projection, and Falcon-H1 with its RMS norm off
// gates y by silu(z)):
//
//   ssd_conv1d_silu  packed x | B | C channels [b, l, ch] ->
//                    silu(bias + causal depthwise conv over time), written
//                    straight into the scan's x [b,l,h,p], B and C [b,l,g,n]
//   ssd_gated_norm   y * silu(z), then an RMS norm over groups of channels
//                    times a per-channel weight
//
// Both are bound by HBM: every input element is read once and every output
// element written once, with 4 consecutive channels per lane (8- or 16-byte
// accesses, a wave covering 256 consecutive channels of one token).
#include <hip/hip_runtime.h>

#include "../../include/ssd.h"
#include "ssd_device.hpp"
#include "ssd_plan.hpp"

namespace ssd {

namespace {

// silu(v) = v / (1 + e^-v) from the hardware exp2 and reciprocal (each
// about 1 ulp): a handful of instructions instead of the library exp and a
// full-precision divide, which made both kernels bound by ALU issue.  For
// v << 0, e^-v overflows to inf and the reciprocal to 0 (result -0).
__device__ __forceinline__ float silu_f(float v) {
    return v * __builtin_amdgcn_rcpf(1.f + exp2_fast(-v * kLog2e));
}

// ----------------------------------------------------------------- conv1d --
// One thread: 4 consecutive channels over kConvRun consecutive tokens.  All
// the run's rows and the width - 1 rows before it are requested before any
// arithmetic (bf16 rows stay packed in registers until used), then the
// outputs are formed and stored.  With a document index, a tap whose source
// token lies in another document than the output token reads zero; rows
// before token 0 come from conv_init and belong to token 0's document.
constexpr int kConvRun = 8;
constexpr int kConvThreads = 256;

// 4 io elements as loaded (bf16 stays packed in registers until used)
template <typename IO> struct Raw4;
template <> struct Raw4<float> { typedef f32x4 type; };
template <> struct Raw4<bf16> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 widen4(const f32x4 &v) { return v; }
__device__ __forceinline__ f32x4 widen4(const bf16x4 &v) {
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename IO, int K, bool SEQ>
__global__ __launch_bounds__(kConvThreads) void k_conv1d_silu(
    const IO *__restrict__ xbc, const float *__restrict__ w, const float *__restrict__ bias,
    const float *__restrict__ init, const int32_t *__restrict__ seq, IO *__restrict__ xo,
    IO *__restrict__ Bo, IO *__restrict__ Co, float *__restrict__ fin, int64_t l, int ch, int hp,
    int gn, int apply_silu) {
    typedef typename Raw4<IO>::type R4;
    const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * 4;
    if (c0 >= ch) return;
    const int64_t b = blockIdx.z;
    const int64_t t0 = (int64_t)blockIdx.y * kConvRun;
    const IO *src = xbc + b * l * ch + c0;
    const int32_t *sq = SEQ ? seq + b * l : nullptr;

    // the run's tokens t0 .. t0 + kConvRun - 1 (raw), then the K - 1 before
    // them (fp32: they may come from conv_init), all requested before use
    constexpr int H = K - 1;
    R4 row[kConvRun];
#pragma unroll
    for (int i = 0; i < kConvRun; ++i) {
        const int64_t t = t0 + i;
        if (t < l) row[i] = *reinterpret_cast<const R4 *>(src + t * ch);
        else row[i] = R4{};
    }
    f32x4 halo[H > 0 ? H : 1];
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const int64_t s = t0 - H + j;
        if (s >= 0)
            halo[j] = widen4(*reinterpret_cast<const R4 *>(src + s * ch));
        else
            halo[j] = init ? *reinterpret_cast<const f32x4 *>(init + (b * H + H + s) * ch + c0)
                           : zero4();
    }
    int doc[SEQ ? kConvRun + H : 1];
    if constexpr (SEQ) {
#pragma unroll
        for (int j = 0; j < kConvRun + H; ++j) {
            const int64_t s = t0 - H + j;
            doc[j] = sq[s < 0 ? 0 : (s < l ? s : l - 1)];
        }
    }
    f32x4 wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) wk[k][e] = w[(int64_t)(c0 + e) * K + k];
    const f32x4 bv = bias ? *reinterpret_cast<const f32x4 *>(bias + c0) : zero4();

    // destination: x, B or C (channel groups of 4 never straddle them)
    IO *dst;
    int64_t ds;
    if (c0 < hp) {
        dst = xo + b * l * hp + c0;
        ds = hp;
    } else if (c0 < hp + gn) {
        dst = Bo + b * l * gn + (c0 - hp);
        ds = gn;
    } else {
        dst = Co + b * l * gn + (c0 - hp - gn);
        ds = gn;
    }
    // input j of the window (0 .. kConvRun + H - 1): halo, then the run
    auto in = [&](int j) { return j < H ? halo[j] : widen4(row[j - H]); };
#pragma unroll
    for (int i = 0; i < kConvRun; ++i) {
        const int64_t t = t0 + i;
        if (t < l) {
            f32x4 acc = bv + wk[K - 1] * in(i + H);
#pragma unroll
            for (int k = 0; k < K - 1; ++k)
                if (!SEQ || doc[i + k] == doc[i + H]) acc += wk[k] * in(i + k);
            if (apply_silu)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = silu_f(acc[e]);
            st4(dst + t * ds, acc);
        }
    }
    // the last width - 1 inputs (rows of earlier documents zero), written by
    // the run that ends the sequence
    if (fin && t0 + kConvRun >= l) {
        const int jl = (int)(l - 1 - t0) + H;  // window index of token l - 1
#pragma unroll
        for (int j = 0; j < H; ++j) {
            const int q = jl - H + 1 + j;  // window index of token l - H + j
            f32x4 v = zero4();
#pragma unroll
            for (int r = 0; r < kConvRun + H; ++r)
                if (r == q && (!SEQ || doc[r] == doc[jl])) v = in(r);
            *reinterpret_cast<f32x4 *>(fin + (b * H + j) * ch + c0) = v;
        }
    }
}

// ------------------------------------------------------------- gated norm --
// One wave per (row, channel group).  Groups of up to 256 * kNormVec
// channels are held in registers: every lane requests its y and z vectors at
// once, the sum of squares of v = y * silu(z) is reduced across the wave,
// and v / sqrt(mean(v^2) + eps) * weight is written.  Larger groups take
// two passes over memory (the second from the cache).  y and out may be the
// same buffer: each lane writes only elements it has already read.
constexpr int kNormVec = 8;

template <typename IO>
__device__ __forceinline__ f32x4 gated4(const IO *y, const IO *z, int64_t at) {
    f32x4 v = ld4(y + at);
    if (z) {
        const f32x4 zv = ld4(z + at);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= silu_f(zv[e]);
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <typename IO>
__global__ __launch_bounds__(256) void k_gated_norm(const IO *y, const IO *__restrict__ z,
                                                    const float *__restrict__ w, IO *out,
                                                    int64_t rows, int dim, int G, float eps,
                                                    int normalize) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int ng = dim / G;
    const int64_t r = item / ng;
    if (r >= rows) return;
    const int c0 = (int)(item % ng) * G;
    const int64_t base = r * dim + c0;
    if (G <= 256 * kNormVec) {
        f32x4 v[kNormVec];
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < kNormVec; ++k) {
            const int i = lane * 4 + 256 * k;
            v[k] = i < G ? gated4(y, z, base + i) : zero4();
        }
#pragma unroll
        for (int k = 0; k < kNormVec; ++k)
            ss += v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
        const float scale = normalize ? 1.f / sqrtf(wave_sum(ss) / (float)G + eps) : 1.f;
#pragma unroll
        for (int k = 0; k < kNormVec; ++k) {
            const int i = lane * 4 + 256 * k;
            if (i < G) {
                f32x4 o = v[k] * scale;
                if (normalize && w) o *= *reinterpret_cast<const f32x4 *>(w + c0 + i);
                st4(out + base + i, o);
            }
        }
        return;
    }
    float scale = 1.f;
    if (normalize) {
        float ss = 0.f;
        for (int i = lane * 4; i < G; i += 256) {
            const f32x4 v = gated4(y, z, base + i);
            ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
        scale = 1.f / sqrtf(wave_sum(ss) / (float)G + eps);
    }
    for (int i = lane * 4; i < G; i += 256) {
        f32x4 o = gated4(y, z, base + i) * scale;
        if (normalize && w) o *= *reinterpret_cast<const f32x4 *>(w + c0 + i);
        st4(out + base + i, o);
    }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// dst <- src (or zeros), for a call with no tokens
__global__ void k_copy_or_zero(float *__restrict__ dst, const float *__restrict__ src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

}  // namespace ssd

using namespace ssd;

extern "C" {

int32_t ssd_conv1d_silu(const void *xbc, const float *weight, const float *bias,
                        const float *conv_init, const int32_t *seq_idx, void *x, void *B,
                        void *C, float *conv_final, int64_t batch, int64_t seqlen,
                        int64_t heads, int64_t head_dim, int64_t state_dim, int64_t groups,
                        int64_t width, int32_t apply_silu, int32_t io_dtype, void *hip_stream) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || seqlen < 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0 ||
        groups <= 0 || width < 1)
        return SSD_ERR_SHAPE;
    if (width > 4 || head_dim % 4 != 0 || state_dim % 4 != 0) return SSD_ERR_UNSUPPORTED;
    const int64_t hp = heads * head_dim, gn = groups * state_dim, ch = hp + 2 * gn;
    if (ch > ((int64_t)1 << 24) || batch > 65535 || seqlen > ((int64_t)1 << 36))
        return SSD_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (batch == 0 || seqlen == 0) {
        // nothing to convolve: the window after the sequence is conv_init
        if (conv_final && batch > 0 && width > 1) {
            if (!aligned16(conv_final) || !aligned16(conv_init)) return SSD_ERR_ALIGN;
            const int64_t cnt = batch * (width - 1) * ch;
            hipLaunchKernelGGL(k_copy_or_zero, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0,
                               s, conv_final, conv_init, cnt);
            if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
        }
        return SSD_OK;
    }
    if (!xbc || !weight || !x || !B || !C) return SSD_ERR_NULL;
    if (!aligned16(xbc) || !aligned16(x) || !aligned16(B) || !aligned16(C) ||
        !aligned16(bias) || !aligned16(conv_init) || !aligned16(conv_final) ||
        ((uintptr_t)weight & 3) || ((uintptr_t)seq_idx & 3))
        return SSD_ERR_ALIGN;
    const int64_t runs = (seqlen + kConvRun - 1) / kConvRun;
    if (runs > 65535) return SSD_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((ch / 4 + kConvThreads - 1) / kConvThreads), (unsigned)runs,
                    (unsigned)batch);
    trace_begin(SSD_K_CONV1D, s);
#define SSD_CONV(IO, KK)                                                                       \
    if (seq_idx)                                                                               \
        hipLaunchKernelGGL((k_conv1d_silu<IO, KK, true>), grid, dim3(kConvThreads), 0, s,      \
                           static_cast<const IO *>(xbc), weight, bias, conv_init, seq_idx,     \
                           static_cast<IO *>(x), static_cast<IO *>(B), static_cast<IO *>(C),   \
                           conv_final, seqlen, (int)ch, (int)hp, (int)gn, apply_silu ? 1 : 0); \
    else                                                                                       \
        hipLaunchKernelGGL((k_conv1d_silu<IO, KK, false>), grid, dim3(kConvThreads), 0, s,     \
                           static_cast<const IO *>(xbc), weight, bias, conv_init, nullptr,     \
                           static_cast<IO *>(x), static_cast<IO *>(B), static_cast<IO *>(C),   \
                           conv_final, seqlen, (int)ch, (int)hp, (int)gn, apply_silu ? 1 : 0)
#define SSD_CONV_W(IO)                                                                         \
    switch (width) {                                                                           \
    case 1: SSD_CONV(IO, 1); break;                                                            \
    case 2: SSD_CONV(IO, 2); break;                                                            \
    case 3: SSD_CONV(IO, 3); break;                                                            \
    default: SSD_CONV(IO, 4); break;                                                           \
    }
    if (io_dtype == SSD_BF16) {
        SSD_CONV_W(bf16)
    } else {
        SSD_CONV_W(float)
    }
#undef SSD_CONV_W
#undef SSD_CONV
    trace_end(SSD_K_CONV1D, s);
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

int32_t ssd_gated_norm(const void *y, const void *z, const float *weight, void *out,
                       int64_t rows, int64_t dim, int64_t group_size, float eps,
                       int32_t normalize, int32_t io_dtype, void *hip_stream) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (rows < 0 || dim <= 0 || group_size <= 0 || dim % group_size != 0 || !(eps >= 0.f))
        return SSD_ERR_SHAPE;
    if (group_size % 4 != 0 || dim > ((int64_t)1 << 30)) return SSD_ERR_UNSUPPORTED;
    if (rows == 0) return SSD_OK;
    if (!y || !out) return SSD_ERR_NULL;
    if (!aligned16(y) || !aligned16(z) || !aligned16(out) || !aligned16(weight))
        return SSD_ERR_ALIGN;
    const int64_t waves = rows * (dim / group_size);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > ((int64_t)1 << 31) - 1) return SSD_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    trace_begin(SSD_K_GATED_NORM, s);
    if (io_dtype == SSD_BF16)
        hipLaunchKernelGGL((k_gated_norm<bf16>), dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const bf16 *>(y), static_cast<const bf16 *>(z), weight,
                           static_cast<bf16 *>(out), rows, (int)dim, (int)group_size, eps,
                           normalize ? 1 : 0);
    else
        hipLaunchKernelGGL((k_gated_norm<float>), dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const float *>(y), static_cast<const float *>(z), weight,
                           static_cast<float *>(out), rows, (int)dim, (int)group_size, eps,
                           normalize ? 1 : 0);
    trace_end(SSD_K_GATED_NORM, s);
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
