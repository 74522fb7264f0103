// Host-side launch plan of one ssd_chunk_scan call: sizes, the padded row
// space and the workspace map.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

namespace ssd {

// Rows are processed in blocks of T = 32 rows.  A block never straddles a
// chunk boundary: chunk c owns padded rows
// [c * Qp, (c + 1) * Qp) with Qp = ceil(Q / T) * T; padded rows past the end
// of a chunk or of the sequence carry d = 0 (no write, no decay).
struct ScanPlan {
    int64_t b, l, h, p, n, g;
    int64_t Q;    // tokens per chunk of the computation
    int64_t Qs;   // tokens per chunk of the caller: the chunk states' spacing
    int64_t ns;   // chunk states of the caller (ceil(l / Qs))
    int io;
    int T;        // rows per block
    int64_t nc;   // chunks
    int64_t nsb;  // blocks per chunk (Qp / T)
    int64_t Qp;   // padded rows per chunk
    int64_t lp;   // padded rows per sequence (nc * Qp)
    // workspace offsets (bytes)
    size_t off_lcs, off_dtp, off_wgt, off_sgr, off_hb, off_st, off_lam, off_scl, off_img, off_hc,
        total;
};

// Chunks shorter than one 32-row block are computed as chunks of a whole
// number of them (at least 64 tokens): the kernels pad every chunk to whole
// blocks, so a short chunk would mostly compute on padding.  The result is
// the same up to rounding (the chunk size is a blocking of the same sum);
// the states at the caller's chunk boundaries are then filled in token by
// token from the states at the computed chunks' boundaries.
constexpr int64_t kMinBlockChunk = 32, kFillChunk = 64;
inline int64_t compute_chunk(int64_t Q) {
    return Q >= kMinBlockChunk ? Q : Q * ((kFillChunk + Q - 1) / Q);
}

inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Heads per workgroup of the chunk-state pass and of the chunk output: 128 /
// head_dim (4 for head_dim <= 32) consecutive heads of one group when the
// group size is a multiple of that, else 1.
inline int group_heads(int p, int64_t heads_per_group) {
    const int hp = p >= 64 ? 128 / p : 4;
    return (hp > 1 && heads_per_group % hp == 0) ? hp : 1;
}

// Whether the bf16 chunk output, with workgroups that share B and C over
// several heads, copies its blocks into LDS from fp16 block images (written
// by the state-scan launch) instead of staging them through registers.  The
// images cost one read of B and C and one write of their fp16 copies; they
// pay off where that is small against the x stream (8 g n <= h p).
// SSD_CHUNK_OUT_COPY=0 or 1 in the environment forces either path; both give
// the same results.
inline bool chunk_out_copy(int64_t h, int64_t g, int64_t p, int64_t n) {
    if (const char *e = getenv("SSD_CHUNK_OUT_COPY")) {
        if (e[0] == '0') return false;
        if (e[0] == '1') return true;
    }
    return 8 * g * n <= h * p;
}

// Fills the plan from the sizes; returns false if they are invalid.
inline bool make_plan(ScanPlan &P, int64_t b, int64_t l, int64_t h, int64_t p, int64_t n,
                      int64_t g, int64_t Q, int io) {
    if (b < 0 || l < 0 || h <= 0 || p <= 0 || n <= 0 || g <= 0 || Q <= 0) return false;
    if (h % g != 0) return false;
    P.b = b; P.l = l; P.h = h; P.p = p; P.n = n; P.g = g; P.io = io;
    P.Qs = Q;
    P.Q = compute_chunk(Q);
    P.ns = (l + Q - 1) / Q;
    Q = P.Q;
    P.T = 32;
    P.nc = (l + Q - 1) / Q;
    P.nsb = (Q + P.T - 1) / P.T;
    P.Qp = P.nsb * P.T;
    P.lp = P.nc * P.Qp;
    const int64_t st = n * p;  // elements of one state
    size_t o = 0;
    P.off_lcs = o;  o += align256(b * h * P.lp * 4);
    P.off_dtp = o;  o += align256(b * h * P.lp * 4);
    P.off_wgt = o;  o += align256(b * h * P.lp * 4);
    // packed sequences: every row's last reset row in its block (or -1)
    P.off_sgr = o;  o += align256(b * h * P.lp * 4);
    // boundary states: matrix-core operand type (fp16 for bf16 io, fp32 for
    // fp32 io); room for fp32 so the layout does not depend on the io type
    P.off_hb = o;   o += align256(b * P.nc * h * st * 4);
    P.off_st = o;   o += align256(b * P.nc * h * st * 4);  // chunk states (fp32, or scaled fp16)
    P.off_lam = o;  o += align256(b * h * P.nc * 4);       // chunk log2 decays
    // bf16 io: every chunk state is kept as fp16 times a power-of-two scale
    P.off_scl = o;  o += align256(b * h * P.nc * 4);       // chunk-state scales
    // C and B of every 32-row block of every (batch, chunk, group) as fp16,
    // in the chunk output's LDS layout (bf16 io only; room kept for both)
    P.off_img = o;  o += align256(b * P.nc * g * P.nsb * 2 * P.T * n * 2);
    // fp32 states after the computed chunks, read by the per-token fill
    // (short caller chunks only)
    P.off_hc = o;   o += P.Qs != P.Q ? align256(b * P.nc * h * st * 4) : 0;
    P.total = o;
    return true;
}

struct ScanArgs {
    const void *x, *dt, *B, *C;
    const float *A, *D, *dt_bias;
    int softplus;
    float dt_min, dt_max;
    const float *init;
    void *y;
    float *final_state;
    char *ws;
    const int32_t *seq;  // [b, l] document index of every token, or NULL
    float *states;       // [b, ns, h, n, p] state after every caller chunk, or NULL
    // fp32 io only, or NULL: every token's weight and log2 decay [b, l, h],
    // given in place of the time step (dt, A, dt_bias and the limits unused)
    const float *lw = nullptr, *la = nullptr;
};

struct StepArgs {
    float *state;
    const void *x, *dt, *B, *C;
    const float *A, *D, *dt_bias;
    int softplus;
    float dt_min, dt_max;
    void *y;
    int64_t b, h, p, n, g;
    int io;
};

// Kernel-timing hooks (ssd_trace_*): called around every launch.
void trace_begin(int kernel, hipStream_t s);
void trace_end(int kernel, hipStream_t s);

// States after every caller chunk, stepped token by token from Hc (the fp32
// states after the computed chunks), for caller chunks shorter than the
// computed ones.
hipError_t launch_token_states(const ScanPlan &pl, const ScanArgs &a, const float *Hc,
                               hipStream_t s);

// The fp32 scan dispatched over the compiled (head_dim, state_dim) set.
hipError_t scan_f32(const ScanPlan &pl, const ScanArgs &a, hipStream_t s);

// Launchers, one per (io, head_dim, state_dim) instantiation.
template <typename IO, int P, int N>
hipError_t launch_scan(const ScanPlan &plan, const ScanArgs &a, hipStream_t s);
template <typename IO, int P, int N>
hipError_t launch_step(const StepArgs &a, hipStream_t s);

}  // namespace ssd
