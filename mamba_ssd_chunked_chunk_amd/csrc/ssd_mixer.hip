// The Mamba-2 mixer between its two projections in one call.  The
// transformers issue page on a Mamba-2 layer's paths names a training path
// that runs the split of the projection, the causal conv1d and the chunk
// scan as one fused operation, against an inference path that calls the
// conv and the scan one after the other; the nnterp guide ("Mamba-2" page)
// reads the heads' y before the gated norm and the output projection, and
// gates it by silu(z):
//
//   xbc --conv1d + SiLU + split--> x, B, C --chunk scan--> y --gate, norm--> out
//
// Three passes on one stream and no allocation:
//   1. ssd_conv1d_silu writes x, B and C straight from its registers into
//      the workspace (the split is the store address; no copies);
//   2. the chunk scan reads them there and writes y into `out`;
//   3. the gated norm runs in place on `out`.
// Every argument of the three passes is checked before the first launch.
//
// The passes stay separate kernels on purpose: the scan kernels are bound by
// matrix and vector instruction issue on gfx950, and moving the conv's
// taps and SiLU (on every x element, once per scan kernel that reads it) or
// the gate's SiLU into them costs more issue time than the HBM bytes it
// saves; the conv and the norm are HBM-bound passes whose arithmetic hides
// under their memory time.  The producer-consumer order keeps x, B, C and y
// resident in the 256 MB Infinity Cache between passes at mixer shapes
// whose intermediates fit it.
#include <hip/hip_runtime.h>

#include "../../include/ssd.h"
#include "ssd_plan.hpp"

namespace ssd {
int32_t scan_status(const void *x, const void *dt, const float *A, const void *B, const void *C,
                    const float *D, const float *dt_bias, const float *init_state,
                    const int32_t *seq_idx, const void *y, const float *final_state,
                    const float *chunk_states, int64_t batch, int64_t seqlen, int64_t heads,
                    int64_t head_dim, int64_t state_dim, int64_t groups, int64_t chunk,
                    int32_t io_dtype, const void *workspace, size_t workspace_bytes);
int32_t conv_status(const void *xbc, const float *weight, const float *bias,
                    const float *conv_init, const int32_t *seq_idx, const void *x, const void *B,
                    const void *C, const float *conv_final, int64_t batch, int64_t seqlen,
                    int64_t heads, int64_t head_dim, int64_t state_dim, int64_t groups,
                    int64_t width, int32_t io_dtype);
int32_t norm_status(const void *y, const void *z, const float *weight, const void *out,
                    int64_t rows, int64_t dim, int64_t group_size, float eps, int32_t io_dtype);

namespace {

// Workspace map of one mixer call: the scan's workspace, then x, B and C,
// each at a 256-byte boundary.  false: the sizes overflow.
struct MixerMap {
    size_t scan, x, B, C, total;
};

bool mixer_map(MixerMap &m, int64_t b, int64_t l, int64_t h, int64_t p, int64_t n, int64_t g,
               int64_t chunk, int32_t io_dtype) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return false;
    if (b < 0 || l < 0 || h <= 0 || p <= 0 || n <= 0 || g <= 0 || chunk <= 0) return false;
    const int64_t lim = (int64_t)1 << 56;
    if (b > 0 && l > lim / b) return false;
    const int64_t rows = b * l;
    if (rows > 0 && (h * p > lim / rows || g * n > lim / rows)) return false;
    const int64_t es = io_dtype == SSD_BF16 ? 2 : 4;
    const size_t ws = ssd_chunk_scan_workspace_bytes(b, l, h, p, n, g, chunk);
    if (ws == 0 && rows > 0) return false;
    m.scan = 0;
    m.x = (size_t)align256((int64_t)ws);
    m.B = m.x + (size_t)align256(rows * h * p * es);
    m.C = m.B + (size_t)align256(rows * g * n * es);
    m.total = m.C + (size_t)align256(rows * g * n * es);
    return true;
}

}  // namespace
}  // namespace ssd

using namespace ssd;

extern "C" {

size_t ssd_mixer_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                                 int64_t state_dim, int64_t groups, int64_t chunk,
                                 int32_t io_dtype) {
    MixerMap m;
    if (!mixer_map(m, batch, seqlen, heads, head_dim, state_dim, groups, chunk, io_dtype))
        return 0;
    return m.total;
}

int32_t ssd_mixer_forward(const void *xbc, const void *z, const void *dt,
                          const float *conv_weight, const float *conv_bias, int64_t conv_width,
                          const float *conv_init, float *conv_final, const float *A,
                          const float *D, const float *dt_bias, int32_t dt_softplus,
                          float dt_min, float dt_max, const float *init_state,
                          float *final_state, const int32_t *seq_idx, const float *norm_weight,
                          int64_t norm_group, float eps, int32_t normalize, void *out,
                          int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                          int64_t state_dim, int64_t groups, int64_t chunk, int32_t io_dtype,
                          void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || seqlen < 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0 ||
        groups <= 0 || chunk <= 0 || heads % groups != 0)
        return SSD_ERR_SHAPE;
    MixerMap m;
    if (!mixer_map(m, batch, seqlen, heads, head_dim, state_dim, groups, chunk, io_dtype))
        return SSD_ERR_UNSUPPORTED;
    if (((uintptr_t)workspace & 255) != 0) return SSD_ERR_ALIGN;
    if (!workspace || workspace_bytes < m.total) return SSD_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    void *x = ws + m.x, *B = ws + m.B, *C = ws + m.C;
    const size_t scan_bytes = m.x;
    int32_t st = conv_status(xbc, conv_weight, conv_bias, conv_init, seq_idx, x, B, C, conv_final,
                             batch, seqlen, heads, head_dim, state_dim, groups, conv_width,
                             io_dtype);
    if (st != SSD_OK) return st;
    st = scan_status(x, dt, A, B, C, D, dt_bias, init_state, seq_idx, out, final_state, nullptr,
                     batch, seqlen, heads, head_dim, state_dim, groups, chunk, io_dtype, ws,
                     scan_bytes);
    if (st != SSD_OK) return st;
    const int64_t rows = batch * seqlen, dim = heads * head_dim;
    st = norm_status(out, z, norm_weight, out, rows, dim, norm_group, eps, io_dtype);
    if (st != SSD_OK) return st;

    st = ssd_conv1d_silu(xbc, conv_weight, conv_bias, conv_init, seq_idx, x, B, C, conv_final,
                         batch, seqlen, heads, head_dim, state_dim, groups, conv_width, 1,
                         io_dtype, hip_stream);
    if (st != SSD_OK) return st;
    st = ssd_chunk_scan_ex(x, dt, A, B, C, D, dt_bias, dt_softplus, dt_min, dt_max, init_state,
                           seq_idx, out, final_state, nullptr, batch, seqlen, heads, head_dim,
                           state_dim, groups, chunk, io_dtype, ws, scan_bytes, hip_stream,
                           nullptr);
    if (st != SSD_OK) return st;
    if (!z && !normalize) return SSD_OK;  // the norm pass would copy y onto itself
    return ssd_gated_norm(out, z, norm_weight, out, rows, dim, norm_group, eps, normalize,
                          io_dtype, hip_stream);
}

}  // extern "C"
