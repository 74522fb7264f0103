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

#include <type_traits>

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
// One thread: V consecutive channels (16 bytes of io: 8 bf16 or 4 fp32, or
// 4 bf16 where the x, B, C widths are not multiples of 8) over a segment of
// 32 consecutive tokens.  Threads of a wave take consecutive channel groups
// of one segment, so every row load and store of a wave is one contiguous
// 1 KiB.  With a document index, a tap whose source token lies in another
// document than the output token reads zero; rows before token 0 come from
// conv_init and belong to token 0's document.
constexpr int kConvThreads = 256;
// A thread walks a segment of conv_runs() runs of conv_run() tokens (32
// tokens), its taps held in registers for all of them and the next run's
// rows in flight while one is computed: 4-token runs for 8-channel threads
// (27.0 us at the 130m mixer shape, against 28.9 with 8-token runs and 30.0
// with one 8-token run per thread), 16 for 4-channel ones; an even count
// of runs
template <int V> constexpr int conv_run() { return V == 8 ? 4 : 16; }
template <int V> constexpr int conv_runs() { return V == 8 ? 8 : 2; }

// 4 io elements as loaded (bf16 stays packed in registers until used)
template <typename IO> struct Raw4;
template <> struct Raw4<float> { typedef f32x4 type; };
template <> struct Raw4<bf16> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 widen4(const f32x4 &v) { return v; }
__device__ __forceinline__ f32x4 widen4(const bf16x4 &v) {
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void narrow4(f32x4 &o, const f32x4 &v) { o = v; }
__device__ __forceinline__ void narrow4(bf16x4 &o, const f32x4 &v) {
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
}
// V io elements of one row, moved as one access
template <typename IO, int V> struct alignas(V * sizeof(IO)) RowV {
    typename Raw4<IO>::type q[V / 4];
};

template <typename IO, int K, bool SEQ, int V>
__global__ __launch_bounds__(kConvThreads) void k_conv1d_silu(
    const IO *__restrict__ xbc, const float *__restrict__ w, const float *__restrict__ bias,
    const float *__restrict__ init, const int32_t *__restrict__ seq, IO *__restrict__ xo,
    IO *__restrict__ Bo, IO *__restrict__ Co, float *__restrict__ fin, int64_t l, int ch, int hp,
    int gn, int apply_silu) {
    typedef RowV<IO, V> R;
    constexpr int NQ = V / 4, RUN = conv_run<V>(), NR = conv_runs<V>(), H = K - 1;
    const int ncg = ch / V;
    const int64_t idx = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    const int64_t seg = idx / ncg;
    const int c0 = (int)(idx - seg * ncg) * V;
    const int64_t ts = seg * (RUN * NR);  // the segment's first token
    if (ts >= l) return;
    const int64_t b = blockIdx.y;
    const IO *src = xbc + b * l * ch + c0;
    const int32_t *sq = SEQ ? seq + b * l : nullptr;
    auto clampt = [&](int64_t t) { return t < 0 ? 0 : (t < l ? t : l - 1); };

    // The K - 1 rows before the segment and its first run's rows, then the
    // taps, are all requested before any of them is used: every load reads
    // a clamped, valid row (rows past the end feed no stored output, rows
    // before token 0 are replaced below), so no branch merges a loaded value
    // and the loads stay in flight together.  Each later run's rows are
    // requested before the run before it is computed.
    f32x4 halo[H > 0 ? H : 1][NQ];
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const R r = *reinterpret_cast<const R *>(src + clampt(ts - H + j) * ch);
#pragma unroll
        for (int q = 0; q < NQ; ++q) halo[j][q] = widen4(r.q[q]);
    }
    R ra[RUN], rb[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) ra[i] = *reinterpret_cast<const R *>(src + clampt(ts + i) * ch);
    // document of every window token of the segment
    int doc[SEQ ? NR * RUN + H : 1];
    if constexpr (SEQ) {
#pragma unroll
        for (int j = 0; j < NR * RUN + H; ++j) doc[j] = sq[clampt(ts - H + j)];
    }
    f32x4 wk[K][NQ];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) wk[k][q][e] = w[(int64_t)(c0 + 4 * q + e) * K + k];
    f32x4 bv[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        bv[q] = bias ? *reinterpret_cast<const f32x4 *>(bias + c0 + 4 * q) : zero4();
    // the first segment: the rows before token 0 come from conv_init (or zero)
    if (ts < H) {
#pragma unroll
        for (int j = 0; j < H; ++j) {
            const int64_t s = ts - H + j;
            if (s < 0)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    halo[j][q] = init ? *reinterpret_cast<const f32x4 *>(
                                            init + (b * H + H + s) * ch + c0 + 4 * q)
                                      : zero4();
        }
    }

    // destination: x, B or C (channel groups of V never straddle them)
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
    // Run r of the segment (tokens t0 .. t0 + RUN - 1) from the halo and its
    // rows; afterwards the halo holds its last K - 1 inputs.
    auto run = [&](int r, const R(&row)[RUN]) {
        const int64_t t0 = ts + (int64_t)r * RUN;
        const int dj = r * RUN;  // window index j of this run is doc[dj + j]
        // part q of input j of the window (0 .. RUN + H - 1): halo, then the run
        auto in = [&](int j, int q) { return j < H ? halo[j][q] : widen4(row[j - H].q[q]); };
#pragma unroll
        for (int i = 0; i < RUN; ++i) {
            const int64_t t = t0 + i;
            if (t < l) {
                R o;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    f32x4 acc = bv[q] + wk[K - 1][q] * in(i + H, q);
#pragma unroll
                    for (int k = 0; k < K - 1; ++k)
                        if (!SEQ || doc[dj + i + k] == doc[dj + i + H])
                            acc += wk[k][q] * in(i + k, q);
                    if (apply_silu)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[e] = silu_f(acc[e]);
                    narrow4(o.q[q], acc);
                }
                *reinterpret_cast<R *>(dst + t * ds) = o;
            }
        }
        // the last width - 1 inputs (rows of earlier documents zero),
        // written by the run that ends the sequence
        if (fin && t0 < l && t0 + RUN >= l) {
            const int jl = (int)(l - 1 - t0) + H;  // window index of token l - 1
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const int qi = jl - H + 1 + j;  // window index of token l - H + j
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    f32x4 v = zero4();
#pragma unroll
                    for (int x = 0; x < RUN + H; ++x)
                        if (x == qi && (!SEQ || doc[dj + x] == doc[dj + jl])) v = in(x, q);
                    *reinterpret_cast<f32x4 *>(fin + (b * H + j) * ch + c0 + 4 * q) = v;
                }
            }
        }
        f32x4 nh[H > 0 ? H : 1][NQ];
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
            for (int q = 0; q < NQ; ++q) nh[j][q] = in(RUN + j, q);
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
            for (int q = 0; q < NQ; ++q) halo[j][q] = nh[j][q];
    };
#pragma unroll
    for (int r = 0; r < NR; r += 2) {
#pragma unroll
        for (int i = 0; i < RUN; ++i)
            rb[i] = *reinterpret_cast<const R *>(src + clampt(ts + (r + 1) * RUN + i) * ch);
        run(r, ra);
        if (r + 2 < NR) {
#pragma unroll
            for (int i = 0; i < RUN; ++i)
                ra[i] = *reinterpret_cast<const R *>(src + clampt(ts + (r + 2) * RUN + i) * ch);
        }
        run(r + 1, rb);
    }
}

// ------------------------------------------------------------- gated norm --
// One wave per (row, channel group); 4 consecutive channels per lane, a
// wave covering 256 channels per step.  Groups of up to 256 * NV channels
// (NV <= 8) are held in registers: every lane requests all its y, z and
// weight vectors at once (clamped, valid addresses; lanes past the group's
// end are masked after the loads, so no branch merges a loaded value and
// the loads stay in flight together), the sum of squares of
// v = y * silu(z) is reduced across the wave, and v / sqrt(mean(v^2) + eps)
// * weight is written.  Larger groups take two passes over memory (the
// second from the cache).  y and out may be the same buffer: each lane
// writes only elements its wave has already read.
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

// GATE: z given; NORM: normalize; WT: a weight (with NORM)
template <typename IO, bool GATE, bool NORM, bool WT, int NV>
__global__ __launch_bounds__(256) void k_gated_norm_reg(const IO *y, const IO *__restrict__ z,
                                                        const float *__restrict__ w, IO *out,
                                                        int64_t rows, int dim, int G,
                                                        float eps) {
    typedef typename Raw4<IO>::type R4;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int ng = dim / G;
    const int64_t r = item / ng;
    if (r >= rows) return;
    const int c0 = (int)(item % ng) * G;
    const int64_t base = r * dim + c0;
    R4 ry[NV], rz[GATE ? NV : 1];
    f32x4 wv[WT ? NV : 1];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = lane * 4 + 256 * k;
        const int ii = i < G ? i : 0;
        ry[k] = *reinterpret_cast<const R4 *>(y + base + ii);
        if constexpr (GATE) rz[k] = *reinterpret_cast<const R4 *>(z + base + ii);
        if constexpr (WT) wv[k] = *reinterpret_cast<const f32x4 *>(w + c0 + ii);
    }
    // keep every load above this point (the scheduler would otherwise sink
    // the weight loads to their use after the reduction, each then waited
    // for on its own)
    __builtin_amdgcn_sched_barrier(0);
    f32x4 v[NV];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        v[k] = widen4(ry[k]);
        if constexpr (GATE) {
            const f32x4 zv = widen4(rz[k]);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[k][e] *= silu_f(zv[e]);
        }
        if (lane * 4 + 256 * k >= G) v[k] = zero4();
        ss += v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
    }
    const float scale = NORM ? 1.f / sqrtf(wave_sum(ss) / (float)G + eps) : 1.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = lane * 4 + 256 * k;
        if (i < G) st4(out + base + i, WT ? v[k] * scale * wv[k] : v[k] * scale);
    }
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

// Launches the norm: the register-resident kernel for groups of up to 2048
// channels (NV = 1, 2, 4, 6 or 8 steps of 256), else the two-pass one.
template <typename IO>
hipError_t launch_gated_norm(const IO *y, const IO *z, const float *w, IO *out, int64_t rows,
                             int dim, int G, float eps, bool normalize, dim3 grid,
                             hipStream_t s) {
    const int steps = (G + 255) / 256;
    const bool gate = z != nullptr, wt = normalize && w != nullptr;
    auto go = [&](auto nv_c, auto gate_c, auto norm_c, auto wt_c) {
        constexpr int NV = decltype(nv_c)::value;
        hipLaunchKernelGGL((k_gated_norm_reg<IO, decltype(gate_c)::value,
                                             decltype(norm_c)::value, decltype(wt_c)::value, NV>),
                           grid, dim3(256), 0, s, y, z, w, out, rows, dim, G, eps);
    };
    auto pick = [&](auto nv_c) {
        typedef std::true_type T;
        typedef std::false_type F;
        if (gate) {
            if (!normalize) go(nv_c, T{}, F{}, F{});
            else if (wt) go(nv_c, T{}, T{}, T{});
            else go(nv_c, T{}, T{}, F{});
        } else {
            if (!normalize) go(nv_c, F{}, F{}, F{});
            else if (wt) go(nv_c, F{}, T{}, T{});
            else go(nv_c, F{}, T{}, F{});
        }
    };
    if (steps <= 1) pick(std::integral_constant<int, 1>{});
    else if (steps <= 2) pick(std::integral_constant<int, 2>{});
    else if (steps <= 4) pick(std::integral_constant<int, 4>{});
    else if (steps <= 6) pick(std::integral_constant<int, 6>{});
    else if (steps <= 8) pick(std::integral_constant<int, 8>{});
    else
        hipLaunchKernelGGL((k_gated_norm<IO>), grid, dim3(256), 0, s, y, z, w, out, rows, dim, G,
                           eps, normalize ? 1 : 0);
    return hipGetLastError();
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// dst <- src (or zeros), for a call with no tokens
__global__ void k_copy_or_zero(float *__restrict__ dst, const float *__restrict__ src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

// Every argument check of ssd_conv1d_silu, in its order (SSD_OK: the call
// launches, or has nothing to launch); the mixer runs it before its first
// launch.
int32_t conv_status(const void *xbc, const float *weight, const float *bias,
                    const float *conv_init, const int32_t *seq_idx, const void *x, const void *B,
                    const void *C, const float *conv_final, int64_t batch, int64_t seqlen,
                    int64_t heads, int64_t head_dim, int64_t state_dim, int64_t groups,
                    int64_t width, int32_t io_dtype) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || seqlen < 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0 ||
        groups <= 0 || width < 1)
        return SSD_ERR_SHAPE;
    if (width > 4 || head_dim % 4 != 0 || state_dim % 4 != 0) return SSD_ERR_UNSUPPORTED;
    const int64_t hp = heads * head_dim, gn = groups * state_dim, ch = hp + 2 * gn;
    if (ch > ((int64_t)1 << 24) || batch > 65535 || seqlen > ((int64_t)1 << 36))
        return SSD_ERR_UNSUPPORTED;
    if (batch == 0 || seqlen == 0) {
        if (conv_final && batch > 0 && width > 1 &&
            (!aligned16(conv_final) || !aligned16(conv_init)))
            return SSD_ERR_ALIGN;
        return SSD_OK;
    }
    if (!xbc || !weight || !x || !B || !C) return SSD_ERR_NULL;
    if (!aligned16(xbc) || !aligned16(x) || !aligned16(B) || !aligned16(C) ||
        !aligned16(bias) || !aligned16(conv_init) || !aligned16(conv_final) ||
        ((uintptr_t)weight & 3) || ((uintptr_t)seq_idx & 3))
        return SSD_ERR_ALIGN;
    if (seqlen > ((int64_t)1 << 19)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Every argument check of ssd_gated_norm, in its order.
int32_t norm_status(const void *y, const void *z, const float *weight, const void *out,
                    int64_t rows, int64_t dim, int64_t group_size, float eps, int32_t io_dtype) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (rows < 0 || dim <= 0 || group_size <= 0 || dim % group_size != 0 || !(eps >= 0.f))
        return SSD_ERR_SHAPE;
    if (group_size % 4 != 0 || dim > ((int64_t)1 << 30)) return SSD_ERR_UNSUPPORTED;
    if (rows == 0) return SSD_OK;
    if (!y || !out) return SSD_ERR_NULL;
    if (!aligned16(y) || !aligned16(z) || !aligned16(out) || !aligned16(weight))
        return SSD_ERR_ALIGN;
    const int64_t blocks = (rows * (dim / group_size) + 3) / 4;
    if (blocks > ((int64_t)1 << 31) - 1) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

}  // namespace ssd

using namespace ssd;

extern "C" {

int32_t ssd_conv1d_silu(const void *xbc, const float *weight, const float *bias,
                        const float *conv_init, const int32_t *seq_idx, void *x, void *B,
                        void *C, float *conv_final, int64_t batch, int64_t seqlen,
                        int64_t heads, int64_t head_dim, int64_t state_dim, int64_t groups,
                        int64_t width, int32_t apply_silu, int32_t io_dtype, void *hip_stream) {
    const int32_t st = conv_status(xbc, weight, bias, conv_init, seq_idx, x, B, C, conv_final,
                                   batch, seqlen, heads, head_dim, state_dim, groups, width,
                                   io_dtype);
    if (st != SSD_OK) return st;
    const int64_t hp = heads * head_dim, gn = groups * state_dim, ch = hp + 2 * gn;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (batch == 0 || seqlen == 0) {
        // nothing to convolve: the window after the sequence is conv_init
        if (conv_final && batch > 0 && width > 1) {
            const int64_t cnt = batch * (width - 1) * ch;
            hipLaunchKernelGGL(k_copy_or_zero, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0,
                               s, conv_final, conv_init, cnt);
            if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
        }
        return SSD_OK;
    }
    // 16-byte rows per thread: 8 bf16 channels where x, B and C split at
    // multiples of 8, else 4
    const bool v8 = io_dtype == SSD_BF16 && hp % 8 == 0 && gn % 8 == 0;
    const int V = v8 ? 8 : 4;
    const int64_t seg = v8 ? conv_run<8>() * conv_runs<8>() : conv_run<4>() * conv_runs<4>();
    const int64_t runs = (seqlen + seg - 1) / seg;
    const dim3 grid((unsigned)((ch / V * runs + kConvThreads - 1) / kConvThreads),
                    (unsigned)batch);
#define SSD_CONV(IO, KK, VV)                                                                   \
    if (seq_idx)                                                                               \
        hipLaunchKernelGGL((k_conv1d_silu<IO, KK, true, VV>), grid, dim3(kConvThreads), 0, s,  \
                           static_cast<const IO *>(xbc), weight, bias, conv_init, seq_idx,     \
                           static_cast<IO *>(x), static_cast<IO *>(B), static_cast<IO *>(C),   \
                           conv_final, seqlen, (int)ch, (int)hp, (int)gn, apply_silu ? 1 : 0); \
    else                                                                                       \
        hipLaunchKernelGGL((k_conv1d_silu<IO, KK, false, VV>), grid, dim3(kConvThreads), 0, s, \
                           static_cast<const IO *>(xbc), weight, bias, conv_init, nullptr,     \
                           static_cast<IO *>(x), static_cast<IO *>(B), static_cast<IO *>(C),   \
                           conv_final, seqlen, (int)ch, (int)hp, (int)gn, apply_silu ? 1 : 0)
#define SSD_CONV_W(IO, VV)                                                                     \
    switch (width) {                                                                           \
    case 1: SSD_CONV(IO, 1, VV); break;                                                        \
    case 2: SSD_CONV(IO, 2, VV); break;                                                        \
    case 3: SSD_CONV(IO, 3, VV); break;                                                        \
    default: SSD_CONV(IO, 4, VV); break;                                                       \
    }
    if (io_dtype == SSD_BF16) {
        if (v8) {
            SSD_CONV_W(bf16, 8)
        } else {
            SSD_CONV_W(bf16, 4)
        }
    } else {
        SSD_CONV_W(float, 4)
    }
#undef SSD_CONV_W
#undef SSD_CONV
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

int32_t ssd_gated_norm(const void *y, const void *z, const float *weight, void *out,
                       int64_t rows, int64_t dim, int64_t group_size, float eps,
                       int32_t normalize, int32_t io_dtype, void *hip_stream) {
    const int32_t st = norm_status(y, z, weight, out, rows, dim, group_size, eps, io_dtype);
    if (st != SSD_OK) return st;
    if (rows == 0) return SSD_OK;
    const int64_t waves = rows * (dim / group_size);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > ((int64_t)1 << 31) - 1) return SSD_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const dim3 grid((unsigned)blocks);
    const hipError_t e =
        io_dtype == SSD_BF16
            ? launch_gated_norm<bf16>(static_cast<const bf16 *>(y), static_cast<const bf16 *>(z),
                                      weight, static_cast<bf16 *>(out), rows, (int)dim,
                                      (int)group_size, eps, normalize != 0, grid, s)
            : launch_gated_norm<float>(static_cast<const float *>(y),
                                       static_cast<const float *>(z), weight,
                                       static_cast<float *>(out), rows, (int)dim,
                                       (int)group_size, eps, normalize != 0, grid, s);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
