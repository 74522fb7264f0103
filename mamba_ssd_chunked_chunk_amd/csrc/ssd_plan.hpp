// Host-side launch plan of one ssd_chunk_scan call: sizes, the padded row
// space and the workspace map.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>
#include <stdint.h>

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
        off_hs, off_imx, total;
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

// Whether the fp32 chunk output, with workgroups that share B and C over
// several heads, copies its blocks into LDS from fp16 block images.  The fp32
// path stages through registers; only bf16 io ever copied, and it now has
// kernels of its own.
inline bool chunk_out_copy(int64_t, int64_t, int64_t, int64_t) { return false; }

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
    // (no block images any more: kept as an empty part of the map)
    P.off_img = o;
    // fp32 states after the computed chunks, read by the per-token fill
    // (short caller chunks only)
    P.off_hc = o;   o += P.Qs != P.Q ? align256(b * P.nc * h * st * 4) : 0;
    // bf16 io: the boundary states' scales [b, h, nc] and the initial
    // state's largest magnitude per (batch, head)
    P.off_hs = o;   o += align256(b * h * P.nc * 4);
    P.off_imx = o;  o += align256(b * h * 4);
    P.total = o;
    return true;
}

// Heads per work item of the bf16 chunk-state and chunk-output kernels:
// four heads of a group (two at head_dim 128) where the heads per group
// allow it, else one.
inline int bf16_item_heads(int64_t p, int64_t h, int64_t g) {
    const int hp = p >= 128 ? 2 : 4;
    return (h / g) % hp == 0 ? hp : 1;
}

int device_cus();

// The interval, in caller chunks, between the states the three bf16 passes
// hand to each other.  The chunk-state pass and the chunk output walk a
// chunk in 32-row blocks with a running state, so a chunk's length costs no
// extra arithmetic: it sets only how many states are stored, scanned and
// read back (each once) and how many work items the two parallel passes
// have.  Where the caller asks for no state after every chunk, the largest
// of 8, 4 and 2 consecutive chunks of the caller is computed as one that
// still leaves two or more workgroups per compute unit (the grid then fills
// the chip at least once at two resident workgroups each), which divides
// the state traffic by as much; no longer join where a shorter one already
// covers the whole sequence.  It is the same sum over the same blocks, with
// fewer states rounded to their stored type on the way.  hp: heads per work
// item.
inline int state_interval(const ScanPlan &pl, bool per_chunk_states, int hp) {
    if (per_chunk_states || pl.Q % 32 != 0) return 1;
    const int64_t want = 2 * (int64_t)device_cus();
    for (int m = 8; m > 1; m /= 2) {
        if ((pl.l + (m / 2) * pl.Q - 1) / ((m / 2) * pl.Q) == 1) continue;
        const int64_t nc = (pl.l + m * pl.Q - 1) / (m * pl.Q);
        if (pl.b * nc * (pl.h / hp) >= want) return m;
    }
    return 1;
}

// The state interval the bf16 scan runs a call at.  Head_dim 64 with a
// group's heads in fours (the four-head workgroups) may instead take the
// split layout's own interval (two heads of two waves per workgroup, three
// workgroups per compute unit): where the split items at that interval fit
// the chip in one round while the four-head grid at its interval does not
// (mamba2_2p7b: 640 split items of 4 joined chunks against 640 four-head
// items of 2 in 1.25 rounds; 0.247 -> 0.235 ms on one box).  may_split:
// not for the gradient pass's row-dot scans nor given boundary states.
inline int bf16_state_interval(const ScanPlan &pl, bool per_chunk_states, int64_t p,
                               bool may_split) {
    const int hpg = bf16_item_heads(p, pl.h, pl.g);
    int m = state_interval(pl, per_chunk_states, hpg);
    if (p == 64 && hpg == 4 && may_split) {
        const int ms = state_interval(pl, per_chunk_states, 2);
        const int64_t cap = 3 * (int64_t)device_cus();
        auto split_items = [&](int mm) {
            return 2 * pl.b * ((pl.l + pl.Q * mm - 1) / (pl.Q * mm)) * (pl.h / 4);
        };
        if (ms > m && split_items(ms) <= cap && split_items(m) > cap) m = ms;
    }
    return m;
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
    // bf16 io only (the gradient pass's scans; defaults give the forward):
    //   xrow  row stride of x in elements (0: heads * head_dim);
    //   xdiv  heads per x slot: head hh reads x slot hh / xdiv (a group's
    //         row of a [b, l, groups, width] tensor for xdiv = heads/groups);
    //   adj   every row's weight is 1 instead of its time step, and the
    //         sequence's first row takes no decay (the adjoint recurrence
    //         g_t = alpha_{t+1} g_{t+1} + C_t dy_t^T, run on reversed rows
    //         whose time steps are the next token's);
    //   dotv  NULL, or (one head per workgroup only) a [b, l, slots, P]
    //         tensor in the io type, row stride dotrow elements, head hh
    //         reading slot hh / dotdiv: the chunk output then also writes
    //         every output row's dot with its row, from the fp32 values
    //         before rounding, to dotout [b, l, heads, waves per head] (one
    //         part per wave's columns)
    int64_t xrow = 0;
    int xdiv = 1;
    int adj = 0;
    const void *dotv = nullptr;
    int64_t dotrow = 0;
    int dotdiv = 1;
    float *dotout = nullptr;
    //   interval  caller chunks per computed chunk (0: state_interval's
    //             choice)
    //   hb_in     NULL, or the boundary states (scaled fp16) and their
    //   hs_in     scales of an earlier call with the same chunks: only the
    //             chunk output runs, reading them; hbt: they hold the
    //             transposed states ([state_dim][head_dim] order of this
    //             call's state)
    //   rev       the call's row t is the tensors' row l - 1 - t (x, B, C,
    //             dt (row l - 1 - t + dshift, past the end: zero), seq and
    //             the outputs y and dotout): a recurrence run backwards in
    //             time without reversed copies
    int rev = 0, dshift = 0;
    int interval = 0;
    const void *hb_in = nullptr;
    const float *hs_in = nullptr;
    int hbt = 0;
    // NULL, or 2 * kEventSlots hipEvent_t owned by the caller: the start and
    // end of the call's launch in each slot (kernel execution only), see
    // launch_timed
    void *const *ev = nullptr;
};

// Slots of the kernel-timing events of one scan call.
enum { kSlotState = 0, kSlotScan = 1, kSlotOut = 2, kSlotFill = 3, kEventSlots = 4 };

// Launches a kernel on stream s, recording events ev[2 slot] and
// ev[2 slot + 1] (when ev is given) at its start and end: the runtime takes
// them from the dispatch itself, so they measure the kernel alone.
template <typename... KArgs, typename... Args>
inline hipError_t launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                               void *const *ev, int slot, Args... args) {
    hipEvent_t e0 = ev ? static_cast<hipEvent_t>(ev[2 * slot]) : nullptr;
    hipEvent_t e1 = ev ? static_cast<hipEvent_t>(ev[2 * slot + 1]) : nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, static_cast<KArgs>(args)...);
    return hipGetLastError();
}

// Compute units of the current device and resident workgroups of a kernel
// per compute unit, queried once per device (thread-safe caches).
int device_cus();
template <auto KERN> int resident_per_cu(int threads) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, KERN, threads, 0) != hipSuccess ||
        nb < 1)
        nb = 1;
    cache[dev].store(nb, std::memory_order_relaxed);
    return nb;
}

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

// States after every caller chunk, stepped token by token from Hc (the fp32
// states after the computed chunks), for caller chunks shorter than the
// computed ones.
hipError_t launch_token_states(const ScanPlan &pl, const ScanArgs &a, const float *Hc,
                               hipStream_t s);

// The fp32 scan dispatched over the compiled (head_dim, state_dim) set.
hipError_t scan_f32(const ScanPlan &pl, const ScanArgs &a, hipStream_t s);
// the bf16 scan kernels (ScanArgs' xrow / xdiv / adj / dot modes)
hipError_t scan_bf16(const ScanPlan &pl, const ScanArgs &a, hipStream_t s);

// Launchers, one per (io, head_dim, state_dim) instantiation.
template <typename IO, int P, int N>
hipError_t launch_scan(const ScanPlan &plan, const ScanArgs &a, hipStream_t s);
template <int P, int N>
hipError_t launch_scan16(const ScanPlan &plan, const ScanArgs &a, hipStream_t s);
template <typename IO, int P, int N>
hipError_t launch_step(const StepArgs &a, hipStream_t s);

}  // namespace ssd
