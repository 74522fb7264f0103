/*
 * ssd.h -- C ABI of libssd.so: the Mamba-2 SSD selective-state-space scan on
 * AMD MI355X (gfx950).
 *
 * Entry points: the chunked scan (ssd_chunk_scan, ssd_chunk_scan_ex with
 * packed documents and the state after every chunk or token,
 * ssd_chunk_scan_noalloc on the library's own scratch), the decode
 * step (ssd_step), the steps just before and after the scan in a Mamba-2
 * mixer (ssd_conv1d_silu, ssd_gated_norm, and both with the scan in one call:
 * ssd_mixer_forward), the deterministic gradient pass
 * (ssd_chunk_scan_bwd), and the pieces of a sequence split into segments
 * (ssd_segment_log_decay, ssd_combine_segments); plus workspace queries
 * and status strings.
 *
 * The scan (nnterp guide, "Mamba-2" page, opening section): per head the
 * state h is a state_dim x head_dim matrix, and every token t does
 *
 *     h = exp(A d_t) h + d_t B_t x_t^T          (decay, then write)
 *     y_t = C_t^T h + D x_t                      (read after the write)
 *
 * where d_t is the processed time step of section "The values":
 * d_t = clamp(softplus(dt_t + dt_bias), dt_min, dt_max) (softplus optional).
 * The heads of a group share B and C; head hh uses group hh / (heads/groups).
 *
 * Layouts (section "The values"; all row-major and contiguous):
 *   x   [batch, seqlen, heads, head_dim]        io dtype
 *   dt  [batch, seqlen, heads]                  io dtype (raw, before bias)
 *   B,C [batch, seqlen, groups, state_dim]      io dtype
 *   A, D, dt_bias [heads]                       fp32
 *   states [batch, heads, state_dim, head_dim]  fp32 (state_dim first)
 *   y   [batch, seqlen, heads, head_dim]        io dtype
 * A decode step drops the seqlen axis (section "The state between steps").
 *
 * Every pointer argument except the stream is a device pointer.  The caller
 * owns every buffer; the library allocates nothing (ssd_chunk_scan_noalloc
 * uses a static device array the library holds instead of a workspace).  Calls are asynchronous
 * on the given HIP stream (NULL = the null stream) and never synchronise.
 * Arguments are validated before anything is launched: a call that returns
 * an error has launched nothing and left every output untouched.  A device
 * fault surfaces at the caller's next synchronisation.  No C++ exception
 * crosses this interface.
 *
 * Preconditions not checked on the device: A <= 0 (decays are non-positive,
 * section "The values"), inputs finite, y not overlapping any input.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 6

/* io dtype of x, dt, B, C and y */
enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1 };

enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = -2,       /* a size < 0 (or <= 0 where a size of 0 is meaningless),
                                 heads % groups != 0, chunk <= 0 */
    SSD_ERR_UNSUPPORTED = -3, /* head_dim / state_dim outside the compiled set, or
                                 an io dtype other than SSD_F32 / SSD_BF16 */
    SSD_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than the query returns */
    SSD_ERR_ALIGN = -5,       /* a pointer is not aligned as documented */
    SSD_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
    SSD_ERR_SCRATCH = -7      /* ssd_chunk_scan_noalloc: the sizes need more scratch
                                 than SSD_SCRATCH_BYTES */
};

/*
 * ssd_chunk_scan -- the prompt / forward scan over a whole sequence.
 *
 * Computes the recurrence above for every (batch, head) from init_state (or
 * from zero) in the chunked two-stage form (kongchang "Mamba2" page,
 * chunk-scan entry: parallel inside a chunk, serial across chunks).  The
 * state at every chunk boundary is kept in the workspace as one tensor
 * (nnterp, "The state after every token": the chunk scan holds the state at
 * each chunk boundary, each a cumulative function of the initial state).
 * The result equals the token-by-token recurrence up to rounding order.
 *
 *   x, dt, B, C   inputs in io_dtype (layouts above); x, B, C 16-byte aligned
 *   A             [heads] fp32, required
 *   D             [heads] fp32, NULL -> no skip term
 *   dt_bias       [heads] fp32, NULL -> zero bias
 *   dt_softplus   nonzero -> d = softplus(dt + dt_bias), else d = dt + dt_bias
 *   dt_min,dt_max time-step limit applied after the softplus (use 0, +INF
 *                 for none)
 *   init_state    [batch, heads, state_dim, head_dim] fp32 or NULL (zeros);
 *                 16-byte aligned
 *   y             output, io dtype, written for every token; 16-byte aligned
 *   final_state   output [batch, heads, state_dim, head_dim] fp32 or NULL (not
 *                 written); may equal init_state (in-place continuation);
 *                 16-byte aligned
 *   chunk         chunk length (any value >= 1; boundary states every chunk
 *                 tokens; the last chunk may be shorter).  A chunk shorter
 *                 than 32 tokens is computed as chunks of a whole number of
 *                 them (the smallest multiple >= 64 tokens): the same sum in
 *                 a coarser blocking, equal up to rounding.
 *   workspace     device scratch of at least ssd_chunk_scan_workspace_bytes
 *                 (...) bytes, 256-byte aligned; contents on entry ignored
 *   hip_stream    hipStream_t to launch on
 *
 * Supported: head_dim in {16, 32, 64, 128}, state_dim in {32, 64, 128}.
 * batch == 0 or seqlen == 0 is valid: nothing is computed except that
 * final_state (if given) receives init_state, or zeros.
 *
 * Precision (bf16 io): the matrix products run on bf16 matrix-core
 * instructions with fp32 accumulation.  x, B and C enter them exactly as
 * given (any finite bf16 value).  Each operand formed inside the scan (the
 * decay-weighted x, the masked scores with the skip term, the carried state)
 * is an fp32 value v split into two bf16 terms, bf16(v) and bf16(v - bf16(v)),
 * both multiplied: 16 significant bits with fp32's exponent range.  Every
 * chunk's own state and the state entering every chunk are kept in the
 * workspace as fp16 times a power of two per (batch, chunk, head) chosen so
 * that nothing overflows (11 significant bits relative to the largest
 * magnitude).  The recurrence across chunks, all sums and decays, and
 * final_state are fp32; y is rounded to nearest even.
 * fp32 io uses fp32 operands and fp32 boundary states throughout.
 */
int32_t ssd_chunk_scan(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const float *dt_bias,
                       int32_t dt_softplus, float dt_min, float dt_max,
                       const float *init_state, void *y, float *final_state,
                       int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                       int64_t state_dim, int64_t groups, int64_t chunk, int32_t io_dtype,
                       void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * ssd_chunk_scan_ex -- ssd_chunk_scan with packed sequences and the state
 * after every chunk.  ssd_chunk_scan is this call with both new pointers
 * NULL; every other argument, the workspace and the error behaviour are
 * the same.
 *
 *   seq_idx       [batch, seqlen] int32 document index of every token, or
 *                 NULL; 4-byte aligned.  Wherever it changes from one token
 *                 to the next, the later token starts from a zero state
 *                 (documents packed into one row; the sample-packing reset
 *                 of the Mamba2 news page).  The initial state, if given,
 *                 belongs to the row's first document; the final state is
 *                 the last document's.  Only whether neighbouring values are
 *                 equal matters.
 *   chunk_states  output [batch, chunks, heads, state_dim, head_dim] fp32, or
 *                 NULL; 16-byte aligned; chunks = ceil(seqlen / chunk).
 *                 Entry c is the state after the last token of chunk c
 *                 (nnterp guide, "The state after every token": one state
 *                 per chunk boundary; chunk = 1 gives the state after every
 *                 token, and the last entry is the final state).  For a
 *                 chunk shorter than 32 tokens the states are stepped token
 *                 by token (fp32) from the states at the computed chunks'
 *                 boundaries, in one extra launch; the last entry then
 *                 equals final_state up to rounding only.
 *   kernel_events NULL, or 8 hipEvent_t created by the caller (hipEventCreate):
 *                 entries 2k and 2k + 1 receive the start and end of the
 *                 call's kernel in slot k -- 0: the chunk-state pass, 1: the
 *                 serial pass over chunks, 2: the chunk output, 3: the
 *                 per-token state fill (only for chunks shorter than 32
 *                 tokens with chunk_states) -- taken from the dispatch
 *                 itself, so an event pair measures that kernel alone.
 *                 Entries may be NULL; a slot the call does not launch is not
 *                 recorded.  The events stay owned by the caller.
 */
int32_t ssd_chunk_scan_ex(const void *x, const void *dt, const float *A, const void *B,
                          const void *C, const float *D, const float *dt_bias,
                          int32_t dt_softplus, float dt_min, float dt_max,
                          const float *init_state, const int32_t *seq_idx, void *y,
                          float *final_state, float *chunk_states, int64_t batch,
                          int64_t seqlen, int64_t heads, int64_t head_dim, int64_t state_dim,
                          int64_t groups, int64_t chunk, int32_t io_dtype, void *workspace,
                          size_t workspace_bytes, void *hip_stream, void *const *kernel_events);

/*
 * Bytes of workspace ssd_chunk_scan needs for these sizes (a pure function
 * of its arguments; 0 for invalid sizes).  Layout, in order, each part
 * 256-byte aligned (the same for both io dtypes; parts an io dtype does not
 * use are left alone): four per-row arrays [batch, heads, padded seqlen] fp32
 * (fp32 io: cumulative log2 decay inside 32-row blocks, processed time step,
 * weight in the state at the block end, packed-sequence reset row);
 * chunk-boundary states [batch, chunks, heads, head_dim, state_dim]
 * (transposed; fp32 for fp32 io, scaled fp16 for bf16 io); every chunk's own
 * state from zero, same shape and types; the log2 decay of every chunk
 * [batch, heads, chunks] fp32; the chunk states' largest magnitudes (bf16)
 * or scales, same shape; for chunks shorter than 32 tokens with
 * chunk_states, the fp32 states after the computed chunks; the boundary
 * states' scales [batch, heads, chunks] and the initial state's largest
 * magnitude per (batch, head) (bf16 io).  Contents on entry are ignored.
 */
size_t ssd_chunk_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads,
                                      int64_t head_dim, int64_t state_dim,
                                      int64_t groups, int64_t chunk);

/*
 * Number of chunks per sequence whose boundary states one ssd_chunk_scan or
 * ssd_chunk_scan_ex call with these sizes computes, stores and scans on the
 * current HIP device: the caller's chunks (ceil(seqlen / chunk), or the
 * coarser computed chunks of a chunk shorter than 32 tokens), except that
 * the bf16 scan computes runs of 8, 4 or 2 of the caller's chunks as one
 * chunk when it asks for no state after every chunk and the chunk is a
 * multiple of 32 tokens: the longest run after which the two parallel
 * passes still have at least two workgroups per compute unit of the device
 * (none longer than a shorter run that already covers the whole sequence).
 * Each computed chunk is the same sum over
 * the same 32-row blocks (kongchang "Mamba2" page, chunk-scan entry: the
 * chunk length is a blocking of the one recurrence), so only the number of
 * stored states changes.  The workspace's state arrays are then filled for
 * that many chunks (a prefix of the layout ssd_chunk_scan_workspace_bytes
 * sizes for the caller's chunks).
 *   with_chunk_states  nonzero if the call passes chunk_states
 * Returns the count (>= 0), or SSD_ERR_SHAPE / SSD_ERR_UNSUPPORTED for sizes
 * or an io dtype the scan rejects.  Queries the device's compute units
 * (once per device); allocates nothing.
 */
int64_t ssd_chunk_scan_state_chunks(int64_t batch, int64_t seqlen, int64_t heads,
                                    int64_t head_dim, int64_t state_dim, int64_t groups,
                                    int64_t chunk, int32_t io_dtype, int32_t with_chunk_states);

/*
 * ssd_chunk_scan_noalloc -- ssd_chunk_scan_ex without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The call
 * allocates nothing (no hipMalloc, no allocating library routine); the
 * scan's scratch is a static device array of SSD_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.
 *
 * Arguments, results, precision and error behaviour are those of
 * ssd_chunk_scan_ex, except that sizes whose ssd_chunk_scan_workspace_bytes
 * (...) exceeds SSD_SCRATCH_BYTES are rejected with SSD_ERR_SCRATCH before
 * anything is launched (128 MiB holds, e.g., 8 x 2048 tokens of 24 heads,
 * head_dim 64, state_dim 128, chunk 256).  All calls on one GPU share its
 * scratch: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.  The scratch's contents are
 * never read before the call writes them.
 */
#define SSD_SCRATCH_BYTES (128u << 20)
int32_t ssd_chunk_scan_noalloc(const void *x, const void *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *dt_bias,
                               int32_t dt_softplus, float dt_min, float dt_max,
                               const float *init_state, const int32_t *seq_idx, void *y,
                               float *final_state, float *chunk_states, int64_t batch,
                               int64_t seqlen, int64_t heads, int64_t head_dim,
                               int64_t state_dim, int64_t groups, int64_t chunk,
                               int32_t io_dtype, void *hip_stream, void *const *kernel_events);

/*
 * ssd_step -- one decode step: no sequence axis, the state updated in place,
 * only y returned (nnterp, "The state between steps").  Exactly one
 * iteration of the recurrence above, with the same time-step processing as
 * ssd_chunk_scan, so a prompt scan followed by steps continues it.
 *
 *   state   [batch, heads, state_dim, head_dim] fp32, read and overwritten;
 *           16-byte aligned
 *   x       [batch, heads, head_dim] io dtype, aligned to 4 elements (16
 *           bytes fp32, 8 bytes bf16); dt [batch, heads] io dtype
 *   B, C    [batch, groups, state_dim] io dtype
 *   A, D, dt_bias, dt_softplus, dt_min, dt_max: as for ssd_chunk_scan
 *   y       [batch, heads, head_dim] io dtype, written; aligned as x
 *
 * With d = 0 (dt_softplus = 0, dt + dt_bias = 0) the state is left exactly
 * unchanged (exp(0) = 1 and nothing is written).
 */
int32_t ssd_step(float *state, const void *x, const void *dt, const float *A,
                 const void *B, const void *C, const float *D, const float *dt_bias,
                 int32_t dt_softplus, float dt_min, float dt_max, void *y, int64_t batch,
                 int64_t heads, int64_t head_dim, int64_t state_dim, int64_t groups,
                 int32_t io_dtype, void *hip_stream);

/*
 * ssd_conv1d_silu -- the short causal convolution in front of the scan, in
 * one pass (the transformers issue page on a Mamba-2 layer's two paths: the
 * causal conv1d, then the chunk scan).  The packed projection channels
 * x | B | C go through a depthwise causal convolution over time, a bias and
 * SiLU, and are written straight into the scan's inputs:
 *
 *   pre[t, c] = bias[c] + sum_{k < width} weight[c, k] * in[t - (width-1) + k, c]
 *   x, B, C   = split(silu(pre))  (silu(v) = v / (1 + exp(-v)); or pre as is
 *                                  with apply_silu = 0)
 *
 *   xbc         [batch, seqlen, ch] io dtype, ch = heads*head_dim +
 *               2*groups*state_dim, channels ordered x (head-major), B, C
 *               (group-major); 16-byte aligned
 *   weight      [ch, width] fp32 (tap width-1 multiplies the current token);
 *               4-byte aligned.  bias [ch] fp32 or NULL; 16-byte aligned
 *   conv_init   [batch, width-1, ch] fp32 inputs before token 0 (oldest
 *               first), or NULL (zeros); 16-byte aligned
 *   seq_idx     [batch, seqlen] int32 document index or NULL: a tap whose
 *               source token lies in another document than the output token
 *               reads zero (conv_init belongs to the first document)
 *   x, B, C     outputs [b,l,h,p], [b,l,g,n], [b,l,g,n] io dtype (bf16
 *               rounded to nearest even); 16-byte aligned
 *   conv_final  output [batch, width-1, ch] fp32 or NULL: the last width-1
 *               inputs (rows of earlier documents zero), the conv_init of a
 *               continuation
 *   width       1..4; head_dim and state_dim multiples of 4
 *
 * fp32 arithmetic.  Errors as for ssd_chunk_scan; SSD_ERR_UNSUPPORTED also
 * for width > 4, more than 65535 batch rows or 2^19 tokens.
 */
int32_t ssd_conv1d_silu(const void *xbc, const float *weight, const float *bias,
                        const float *conv_init, const int32_t *seq_idx, void *x, void *B,
                        void *C, float *conv_final, int64_t batch, int64_t seqlen,
                        int64_t heads, int64_t head_dim, int64_t state_dim, int64_t groups,
                        int64_t width, int32_t apply_silu, int32_t io_dtype, void *hip_stream);

/*
 * ssd_gated_norm -- the steps after the scan, in one pass (nnterp guide: the
 * heads' y is read before the gated norm and the output projection; with
 * Falcon-H1's RMS norm off, y is gated by silu(z)):
 *
 *   v   = y * silu(z)                       (v = y when z is NULL)
 *   out = v / sqrt(mean_group(v^2) + eps) * weight   (normalize != 0;
 *                                            out = v otherwise)
 *
 *   y, z, out   [rows, dim] io dtype (y of [b, l, h, p] is rows = b*l,
 *               dim = h*p); 16-byte aligned; out may equal y
 *   weight      [dim] fp32 or NULL (ones); 16-byte aligned
 *   group_size  channels per norm group (dim % group_size == 0, a multiple
 *               of 4); eps >= 0
 *
 * fp32 arithmetic, bf16 output rounded to nearest even.
 */
int32_t ssd_gated_norm(const void *y, const void *z, const float *weight, void *out,
                       int64_t rows, int64_t dim, int64_t group_size, float eps,
                       int32_t normalize, int32_t io_dtype, void *hip_stream);

/*
 * ssd_mixer_forward -- the Mamba-2 mixer between its two projections in one
 * call: the split of the projection channels, the causal conv1d + SiLU, the
 * chunk scan and the gated RMS norm.  The transformers issue page on a
 * Mamba-2 layer's paths names a training path that runs the split, the conv
 * and the scan as one fused operation against an inference path of separate
 * calls; the nnterp guide ("Mamba-2" page) reads y before the gated norm and
 * the output projection.  The result is, bit for bit, that of
 *
 *   ssd_conv1d_silu(xbc, ... apply_silu = 1) -> x, B, C
 *   ssd_chunk_scan_ex(x, dt, A, B, C, D, dt_bias, ..., seq_idx) -> y
 *   ssd_gated_norm(y, z, norm_weight, out, b*l, h*p, norm_group, eps, normalize)
 *
 * with x, B and C held in the workspace and y written into `out` (the norm
 * then runs in place).  No pass is skipped except the norm when z is NULL
 * and normalize is 0 (out = y).
 *
 *   xbc, conv_weight, conv_bias, conv_width, conv_init, conv_final
 *                 as for ssd_conv1d_silu (conv_init/conv_final may be NULL)
 *   dt, A, D, dt_bias, dt_softplus, dt_min, dt_max, init_state,
 *   final_state, seq_idx
 *                 as for ssd_chunk_scan_ex (seq_idx also masks the conv)
 *   z             [b, l, h*p] io dtype gate or NULL; 16-byte aligned
 *   norm_weight, norm_group, eps, normalize
 *                 as for ssd_gated_norm (norm_group > 0 always)
 *   out           [b, l, h, p] io dtype output; 16-byte aligned; must not
 *                 overlap any input or the workspace
 *   workspace     at least ssd_mixer_workspace_bytes(...) bytes, 256-byte
 *                 aligned: the scan's workspace, then x, B and C
 *
 * Every argument of the three passes is checked before the first launch:
 * an error return has launched nothing (SSD_ERR_HIP aside, which a launch
 * reports after the passes before it were queued).
 */
int32_t ssd_mixer_forward(const void *xbc, const void *z, const void *dt,
                          const float *conv_weight, const float *conv_bias, int64_t conv_width,
                          const float *conv_init, float *conv_final, const float *A,
                          const float *D, const float *dt_bias, int32_t dt_softplus,
                          float dt_min, float dt_max, const float *init_state,
                          float *final_state, const int32_t *seq_idx, const float *norm_weight,
                          int64_t norm_group, float eps, int32_t normalize, void *out,
                          int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                          int64_t state_dim, int64_t groups, int64_t chunk, int32_t io_dtype,
                          void *workspace, size_t workspace_bytes, void *hip_stream);

/* Bytes of workspace ssd_mixer_forward needs (0: invalid or overflowing sizes). */
size_t ssd_mixer_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                                 int64_t state_dim, int64_t groups, int64_t chunk,
                                 int32_t io_dtype);

/*
 * ssd_chunk_scan_bwd -- gradients of ssd_chunk_scan_ex's y and final state,
 * deterministic (every sum in a fixed order; the same inputs give the same
 * bits).  The pages note the backward of the reference kernels is not
 * deterministic (transformers issue page); the gradients here are the exact
 * derivatives of the forward (nnterp guide, "Mamba-2" page recurrence):
 *
 *   adjoint g_t = dL/dh_t = C_t dy_t^T + alpha_{t+1} g_{t+1}  (inside a
 *   document; g of the last token also gets d_final), alpha_t = exp(A d_t)
 *   dx_t = D dy_t + d_t g_t^T B_t,   dB_t = sum_heads d_t g_t x_t,
 *   dC_t = sum_heads h_t dy_t,       da_t = alpha_t <g_t, h_{t-1}>,
 *   ddt_t = (g_t . B_t x_t^T + A da_t) * [dt_min <= softplus(z) <= dt_max]
 *           * sigmoid(z)   (z = dt + dt_bias; without softplus the last
 *           factor is 1),
 *   dA = sum d da,  d dt_bias = sum ddt,  dD = sum dy . x,  d init = alpha_0 g_0.
 *
 *   forward inputs  as for ssd_chunk_scan_ex (init_state, seq_idx optional)
 *   dy              [batch, seqlen, heads, head_dim] io dtype, required
 *   d_final         [batch, heads, state_dim, head_dim] fp32 or NULL (zero)
 *   dx              [b, l, h, p] io dtype          (required)
 *   ddt             [b, l, h] io dtype              (required)
 *   dA              [h] fp32                        (required)
 *   dB, dC          [b, l, g, n] io dtype           (required)
 *   dD, d_dt_bias   [h] fp32 or NULL (not written)
 *   d_init          [b, h, n, p] fp32 or NULL (not written)
 *   workspace       ssd_chunk_scan_bwd_workspace_bytes(...) bytes,
 *                   256-byte aligned
 *
 * Supported: head_dim and state_dim in {32, 64, 128} (the transposed scans
 * take head_dim as their state size).  batch and seqlen >= 1.  The three
 * chunk scans run on the forward's kernels of the io dtype: fp32 io on the
 * fp32 path; bf16 io on the bf16 path (bf16 inputs exact, every derived
 * operand as two bf16 terms, fp32 accumulation; the adjoint scans read the
 * inputs in reversed row order, the transposed scans read each head's
 * group row of B or C, and the sums that need fp32 are taken from the
 * scans' fp32 values before rounding).  The running sums
 * behind ddt, dA, d dt_bias and dD are fp64.  16-byte alignment for x, B,
 * C, dy, dx, dB, dC and the states, element alignment for the rest;
 * SSD_ERR_ALIGN otherwise.  Several launches: three chunk scans and the
 * pass's own kernels.
 */
int32_t ssd_chunk_scan_bwd(const void *x, const void *dt, const float *A, const void *B,
                           const void *C, const float *D, const float *dt_bias,
                           int32_t dt_softplus, float dt_min, float dt_max,
                           const float *init_state, const int32_t *seq_idx, const void *dy,
                           const float *d_final, void *dx, void *ddt, float *dA, void *dB,
                           void *dC, float *dD, float *d_dt_bias, float *d_init, int64_t batch,
                           int64_t seqlen, int64_t heads, int64_t head_dim, int64_t state_dim,
                           int64_t groups, int64_t chunk, int32_t io_dtype, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/* Bytes of workspace ssd_chunk_scan_bwd needs for these sizes and io dtype (0 for
 * invalid sizes or an unknown io dtype). */
size_t ssd_chunk_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads,
                                          int64_t head_dim, int64_t state_dim, int64_t groups,
                                          int64_t chunk, int32_t io_dtype);

/*
 * Sequence segments (one per GPU for contexts beyond one GPU).  The state
 * after a stretch of tokens is a linear function of the state entering it
 * (nnterp guide, "The state after every token"; kongchang "Mamba2" page:
 * states pass serially from chunk to chunk), so a sequence cut into K
 * segments is scanned in two passes:
 *   1. every segment from a zero state (ssd_chunk_scan_ex with final_state):
 *      its own final state S_k; and its total log decay L_k
 *      (ssd_segment_log_decay);
 *   2. ssd_combine_segments: entry_0 = init, entry_{k+1} = exp(L_k) entry_k
 *      + S_k; then every segment again from entry_k: its y and states are
 *      those of one pass over the whole sequence, up to rounding.
 * Across GPUs only the pairs (L_k, S_k) move.
 *
 * ssd_segment_log_decay -- L[b, h] = sum over the segment's tokens of
 *   A[h] * d_t (d_t processed as in ssd_chunk_scan), fp32, summed in fp64
 *   in a fixed order; -INFINITY where a new document starts inside the
 *   segment (after its first token: nothing enters past a reset).
 *   dt [batch, seqlen, heads] io dtype; seq_idx [batch, seqlen] or NULL.
 *
 * ssd_combine_segments -- from log_decay [K, b, h] and seg_states
 *   [K, b, h, n, p] (each segment's final state from a zero state), the
 *   entry state of every segment entry_states [K, b, h, n, p] (or NULL) and
 *   the sequence's final state [b, h, n, p] (or NULL).  init_state
 *   [b, h, n, p] or NULL (zeros).  starts_document [K, b] int32 or NULL:
 *   nonzero where segment k's first token starts a new document in row b
 *   (that segment then takes a zero state in).  fp32, deterministic.
 */
int32_t ssd_segment_log_decay(const void *dt, const float *A, const float *dt_bias,
                              int32_t dt_softplus, float dt_min, float dt_max,
                              const int32_t *seq_idx, float *log_decay, int64_t batch,
                              int64_t seqlen, int64_t heads, int32_t io_dtype,
                              void *hip_stream);
int32_t ssd_combine_segments(const float *log_decay, const float *seg_states,
                             const float *init_state, const int32_t *starts_document,
                             float *entry_states, float *final_state, int64_t segments,
                             int64_t batch, int64_t heads, int64_t head_dim, int64_t state_dim,
                             void *hip_stream);

/* Static text for a status code (never NULL). */
const char *ssd_status_string(int32_t status);

/* SSD_ABI_VERSION of the built library. */
int32_t ssd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
