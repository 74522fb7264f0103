/*
 * ssd_oracle.c -- plain fp64 CPU reference for the Mamba-2 SSD scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes is the definition itself, one token at a time, in fp64
 * (nnterp guide, "Mamba-2" page, opening section): per head the state is a
 * state_dim x head_dim matrix h, and every token does
 *
 *     h = exp(dt * A) * h + dt * B x^T        (write, then decay-and-add)
 *     y = C^T h + D * x                        (read after the write)
 *
 * with dt the processed time step of section "The values" on the same page:
 * dt = softplus(dt_raw + dt_bias), clamped to the time-step limit.  Groups
 * share B and C ("The values": the heads of a group share B and C); head hh
 * uses group hh / (heads / groups).  The state layout is [b, h, n, p], state
 * dim first ("The values": state served key side first).  A decode step is
 * one iteration of the same loop on a carried state (section "The state
 * between steps").  The chunked two-stage form is an exact regrouping of
 * this loop (kongchang "Mamba2" page, chunk-scan entry), so the oracle is
 * the loop, not the chunked algorithm.
 *
 * Inputs are read at their stored precision (fp32, or bf16 bit patterns)
 * and widened exactly to fp64.  libm exp / log1p are used as is.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { IO_F32 = 0, IO_BF16 = 1 };

static double ld(const void *p, int64_t i, int io)
{
    if (io == IO_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[i];
}

/* softplus(z) = log(1 + e^z), written in the overflow-free form. */
static double softplus(double z)
{
    return fmax(z, 0.0) + log1p(exp(-fabs(z)));
}

/* The processed time step of one token (section "The values"). */
static double proc_dt(double raw, double bias, int use_softplus, double lo, double hi)
{
    double z = raw + bias;
    double d = use_softplus ? softplus(z) : z;
    if (d < lo) d = lo;
    if (d > hi) d = hi;
    return d;
}

typedef struct {
    const void *x, *dt, *B, *C;
    const float *A, *D, *dt_bias;
    int softplus, io;
    double dt_min, dt_max;
    const double *init; /* [npairs, n, p] or NULL */
    int64_t b, l, h, p, n, g;
    const int64_t *pairs;
    int64_t npairs;
    double *y;     /* [npairs, l, p] */
    double *state; /* [npairs, n, p] */
    const int32_t *seq_idx; /* [b, l] or NULL */
    int64_t chunk;          /* states output: one state per chunk of this many tokens */
    double *states;         /* [npairs, ceil(l / chunk), n, p] or NULL */
    int64_t next;  /* work counter */
} job_t;

static void run_pair(const job_t *J, int64_t k)
{
    const int64_t bb = J->pairs[2 * k], hh = J->pairs[2 * k + 1];
    const int64_t l = J->l, h = J->h, p = J->p, n = J->n, g = J->g;
    const int64_t gi = hh / (h / g);
    double *H = J->state + k * n * p;
    double *yk = J->y + k * l * p;
    double *xv = (double *)malloc(sizeof(double) * (size_t)(p > 0 ? p : 1));
    const double bias = J->dt_bias ? (double)J->dt_bias[hh] : 0.0;
    const double Ah = (double)J->A[hh];
    const double Dh = J->D ? (double)J->D[hh] : 0.0;

    if (J->init)
        memcpy(H, J->init + k * n * p, sizeof(double) * (size_t)(n * p));
    else
        memset(H, 0, sizeof(double) * (size_t)(n * p));

    for (int64_t t = 0; t < l; ++t) {
        const int64_t row = bb * l + t;
        /* packed sequences: a token whose document index differs from the
           previous token's starts from a zero state */
        if (J->seq_idx && t > 0 && J->seq_idx[row] != J->seq_idx[row - 1])
            memset(H, 0, sizeof(double) * (size_t)(n * p));
        const double d = proc_dt(ld(J->dt, row * h + hh, J->io), bias, J->softplus,
                                 J->dt_min, J->dt_max);
        const double decay = exp(Ah * d);
        for (int64_t j = 0; j < p; ++j)
            xv[j] = ld(J->x, (row * h + hh) * p + j, J->io);
        /* write: h = exp(dt A) h + dt B x^T */
        for (int64_t i = 0; i < n; ++i) {
            const double wb = d * ld(J->B, (row * g + gi) * n + i, J->io);
            double *Hi = H + i * p;
            for (int64_t j = 0; j < p; ++j)
                Hi[j] = decay * Hi[j] + wb * xv[j];
        }
        /* read: y = C^T h + D x */
        double *yt = yk + t * p;
        for (int64_t j = 0; j < p; ++j)
            yt[j] = Dh * xv[j];
        for (int64_t i = 0; i < n; ++i) {
            const double ci = ld(J->C, (row * g + gi) * n + i, J->io);
            const double *Hi = H + i * p;
            for (int64_t j = 0; j < p; ++j)
                yt[j] += ci * Hi[j];
        }
        /* the state after the last token of each chunk */
        if (J->states && ((t + 1) % J->chunk == 0 || t == l - 1)) {
            const int64_t nc = (l + J->chunk - 1) / J->chunk;
            memcpy(J->states + (k * nc + t / J->chunk) * n * p, H,
                   sizeof(double) * (size_t)(n * p));
        }
    }
    free(xv);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    for (;;) {
        int64_t k = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (k >= J->npairs)
            break;
        run_pair(J, k);
    }
    return NULL;
}

/*
 * Runs the recurrence for each requested (batch, head) pair.
 *   x [b,l,h,p], dt [b,l,h], B and C [b,l,g,n] in the io precision
 *   (io 0 = fp32, 1 = bf16 bit patterns); A, D, dt_bias [h] fp32 (D and
 *   dt_bias may be NULL: no skip, zero bias); init [npairs,n,p] fp64 or NULL.
 *   pairs: npairs (b, h) index pairs.
 *   y out [npairs,l,p] fp64; state out [npairs,n,p] fp64.
 *   seq_idx [b,l] int32 or NULL: packed sequences; wherever the index
 *   changes from one token to the next, the later token starts from a zero
 *   state (the initial state belongs to the first sequence of each row).
 *   states out [npairs, ceil(l/chunk), n, p] fp64 or NULL: the state after
 *   the last token of every chunk of `chunk` tokens (nnterp guide, "The
 *   state after every token": one state per chunk boundary; chunk 1 gives
 *   the state after every token, and the last one is the final state).
 * Returns 0, or -1 on a bad argument.
 */
int ssd_oracle_scan(const void *x, const void *dt, const float *A, const void *B,
                    const void *C, const float *D, const float *dt_bias,
                    int dt_softplus, double dt_min, double dt_max, const double *init,
                    int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                    int64_t state_dim, int64_t groups, int io, const int64_t *pairs,
                    int64_t npairs, double *y, double *state, const int32_t *seq_idx,
                    int64_t chunk, double *states, int nthreads)
{
    if (!A || !pairs || !state || (seqlen > 0 && (!x || !dt || !B || !C || !y)))
        return -1;
    if (states && chunk < 1)
        return -1;
    if (batch < 0 || seqlen < 0 || heads <= 0 || head_dim <= 0 || state_dim <= 0 ||
        groups <= 0 || heads % groups != 0 || (io != IO_F32 && io != IO_BF16))
        return -1;
    for (int64_t k = 0; k < npairs; ++k)
        if (pairs[2 * k] < 0 || pairs[2 * k] >= batch || pairs[2 * k + 1] < 0 ||
            pairs[2 * k + 1] >= heads)
            return -1;
    job_t J = {x, dt, B, C, A, D, dt_bias, dt_softplus, io, dt_min, dt_max, init,
               batch, seqlen, heads, head_dim, state_dim, groups, pairs, npairs,
               y, state, seq_idx, chunk, states, 0};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > npairs)
        nthreads = (int)(npairs > 0 ? npairs : 1);
    if (nthreads == 1) {
        worker(&J);
        return 0;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, worker, &J) == 0)
            ++started;
    if (started == 0)
        worker(&J);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    return 0;
}

/* The processed time step d and the log-decay a = A d of every (b, t, h)
 * (section "The values": betas = dt, decays = A * dt). d, a out [b,l,h]. */
int ssd_oracle_dt(const void *dt, const float *A, const float *dt_bias, int dt_softplus,
                  double dt_min, double dt_max, int64_t batch, int64_t seqlen,
                  int64_t heads, int io, double *d_out, double *a_out)
{
    if (!dt || !A || !d_out || !a_out || batch < 0 || seqlen < 0 || heads <= 0)
        return -1;
    for (int64_t r = 0; r < batch * seqlen; ++r)
        for (int64_t hh = 0; hh < heads; ++hh) {
            const double bias = dt_bias ? (double)dt_bias[hh] : 0.0;
            const double d = proc_dt(ld(dt, r * heads + hh, io), bias, dt_softplus,
                                     dt_min, dt_max);
            d_out[r * heads + hh] = d;
            a_out[r * heads + hh] = (double)A[hh] * d;
        }
    return 0;
}
