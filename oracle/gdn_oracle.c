/*
 * CPU oracle for the fused sigmoid-gating + gated delta-rule state update
 * (Gated DeltaNet decode).  TEST INFRASTRUCTURE ONLY: it is called by the
 * tests, by the smoke check and by the benchmark's CPU-baseline leg, never by
 * the product path.  It shares no code with the HIP library.
 *
 * What it computes.  The pages name the operation without printing its
 * equations: vLLM PR #35777 (implementation section) fuses the gating kernel
 * with the recurrent delta-rule update and feeds it A_log, a, b and dt_bias
 * directly, with an rsqrt-based normalisation and a speculative-decoding mode;
 * sglang PR #18271 tiles it over value columns.  The definition written out
 * here is the gated delta rule of Gated DeltaNet, per token t and value head h
 * (k-head j = h / G, G = H_v / H_k):
 *
 *   gamma = exp(-exp(A_log[h]) * softplus(a[t,h] + dt_bias[h]))
 *   beta  = 1 / (1 + exp(-b[t,h]))
 *   khat  = k[t,j] / sqrt(sum k^2 + eps)
 *   qhat  = scale * q[t,j] / sqrt(sum q^2 + eps)        scale = K^-1/2 default
 *   S     = gamma * S                                    (decay)
 *   u     = beta * (v[t,h] - S^T khat)                   (delta)
 *   S     = S + khat u^T                                 (rank-1 update)
 *   o     = S^T qhat                                     (output, post-update S)
 *
 * S is K x V (row index kappa over K, column over V), gathered from
 * pool[state_idx[i], h] and written back there after the sequence's last
 * token.  The pool stores each K x V tile either with V fastest ("KV",
 * element (kappa, c) at kappa*V + c) or transposed with K fastest ("VK",
 * element (kappa, c) at c*K + kappa); intermediate states use the same
 * layout.  Tiles are stored as fp32 or as bf16; a bf16 tile is widened
 * exactly on load and each stored element is the double-precision state
 * rounded straight to the nearest bf16 (ties to even).  Readings where the pages are silent: eps sits inside the square
 * root; a sequence with state_idx < 0 or with no tokens is not touched at all;
 * intermediate_states[t, h] holds S after token t at global token row t.
 *
 * All arithmetic is in double precision with plain loops in the order above.
 * The only rounding to float is the store of S into the fp32 pool and into
 * intermediate_states (C's double->float conversion, round to nearest even).
 * OpenMP runs independent (sequence, v-head) units in parallel; nothing inside
 * a unit is reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_LAYOUT_KV 0
#define ORACLE_LAYOUT_VK 1

#define ORACLE_STATE_F32 0
#define ORACLE_STATE_BF16 1

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* The bit pattern of the bf16 nearest to x (8 significant bits, ties to
 * even), rounded once from double. */
static uint16_t oracle_to_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    double y = x;
    const double ax = fabs(x);
    if (ax != 0.0 && !isinf(x)) {
        if (ax < 0x1p-126) {                /* subnormal range: quantum 2^-133 */
            y = nearbyint(x * 0x1p133) * 0x1p-133;
        } else {
            int e;
            const double m = frexp(x, &e);  /* x = m 2^e, 0.5 <= |m| < 1 */
            y = ldexp(nearbyint(ldexp(m, 8)), e - 8);
        }
    }
    const float f = (float)y;               /* exact (or inf on overflow) */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static double oracle_from_bf16(uint16_t bits)
{
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element e of a state tile stored as fp32 or bf16. */
static double tile_get(const void *tile, size_t e, int bf16)
{
    return bf16 ? oracle_from_bf16(((const uint16_t *)tile)[e]) : (double)((const float *)tile)[e];
}

static void tile_put(void *tile, size_t e, double x, int bf16)
{
    if (bf16)
        ((uint16_t *)tile)[e] = oracle_to_bf16(x);
    else
        ((float *)tile)[e] = (float)x;
}

/* log(1 + e^x) without overflow. */
static double oracle_softplus(double x)
{
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

/* 1 / (1 + e^-x), evaluated on the side that does not overflow. */
static double oracle_sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* Copies x (length n) to y scaled by c / sqrt(sum x^2 + eps). */
static void oracle_l2norm(const double *x, double *y, int n, double eps, double c)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double f = c / sqrt(ss + eps);
    for (int i = 0; i < n; ++i)
        y[i] = x[i] * f;
}

/*
 * q, k      [N, Hk, K]    token rows, dense
 * v, out    [N, Hv, V]
 * a, b      [N, Hv]
 * A_log, dt_bias [Hv]
 * pool      [num_slots, Hv, K, V] fp32, updated in place
 * state_idx [B], -1 (any negative) = padding
 * cu_seqlens [B+1] or NULL (then sequence i owns rows [i*T, (i+1)*T))
 * intermediate [N, Hv, K, V] fp32 or NULL
 * no_final_writeback != 0 leaves the pool unchanged
 * state_layout: ORACLE_LAYOUT_KV or ORACLE_LAYOUT_VK (storage order of the
 *   pool and intermediate tiles)
 * state_dtype: ORACLE_STATE_F32 or ORACLE_STATE_BF16 (pool and intermediates
 *   hold float or bf16 bit patterns)
 * scale <= 0 selects K^-1/2.  threads <= 0 uses the OpenMP default.
 */
int gdn_oracle_update(const double *q, const double *k, const double *v,
                      const double *a, const double *b,
                      const double *A_log, const double *dt_bias,
                      void *pool, const int32_t *state_idx,
                      const int32_t *cu_seqlens, double *out,
                      void *intermediate,
                      int B, int T, int64_t N, int Hk, int Hv, int K, int V,
                      int64_t num_slots, double scale, double eps,
                      int no_final_writeback, int state_layout, int state_dtype,
                      int threads)
{
    if (B < 0 || K <= 0 || V <= 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0)
        return ORACLE_ERR_ARG;
    if (state_layout != ORACLE_LAYOUT_KV && state_layout != ORACLE_LAYOUT_VK)
        return ORACLE_ERR_ARG;
    if (state_dtype != ORACLE_STATE_F32 && state_dtype != ORACLE_STATE_BF16)
        return ORACLE_ERR_ARG;
    const int bf16 = state_dtype == ORACLE_STATE_BF16;
    const size_t esize = bf16 ? 2 : 4;
    /* storage strides of S[kappa][c] inside a tile */
    const size_t row_stride = state_layout == ORACLE_LAYOUT_KV ? (size_t)V : 1;
    const size_t col_stride = state_layout == ORACLE_LAYOUT_KV ? 1 : (size_t)K;
    if (B == 0)
        return ORACLE_OK;
    if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !pool ||
        !state_idx || !out)
        return ORACLE_ERR_ARG;
    if (!cu_seqlens && (T < 0 || (int64_t)B * T > N))
        return ORACLE_ERR_ARG;
    const int G = Hv / Hk;
    const double qscale = scale > 0.0 ? scale : 1.0 / sqrt((double)K);
    const int64_t units = (int64_t)B * Hv;
    int status = ORACLE_OK;

#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic) num_threads(threads)
#endif
    for (int64_t unit = 0; unit < units; ++unit) {
        const int i = (int)(unit / Hv);
        const int h = (int)(unit % Hv);
        const int j = h / G;
        const int32_t slot = state_idx[i];
        if (slot < 0)
            continue;
        if (slot >= num_slots) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = ORACLE_ERR_ARG;
            continue;
        }
        const int64_t t0 = cu_seqlens ? cu_seqlens[i] : (int64_t)i * T;
        const int64_t t1 = cu_seqlens ? cu_seqlens[i + 1] : (int64_t)(i + 1) * T;
        if (t1 <= t0)
            continue;
        if (t0 < 0 || t1 > N) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = ORACLE_ERR_ARG;
            continue;
        }

        double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
        double *kh = (double *)malloc(sizeof(double) * (size_t)K);
        double *qh = (double *)malloc(sizeof(double) * (size_t)K);
        double *u = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !kh || !qh || !u) {
            free(S); free(kh); free(qh); free(u);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = ORACLE_ERR_NOMEM;
            continue;
        }
        char *tile = (char *)pool + ((size_t)slot * Hv + h) * (size_t)K * V * esize;
        for (int kk = 0; kk < K; ++kk)
            for (int c = 0; c < V; ++c)
                S[(size_t)kk * V + c] = tile_get(tile, kk * row_stride + c * col_stride, bf16);

        for (int64_t t = t0; t < t1; ++t) {
            /* gating: decay g and write strength beta */
            const double x = a[t * Hv + h] + dt_bias[h];
            const double g = -exp(A_log[h]) * oracle_softplus(x);
            const double gamma = exp(g);
            const double beta = oracle_sigmoid(b[t * Hv + h]);
            /* L2-normalised key and query of k-head j */
            oracle_l2norm(k + (t * Hk + j) * (int64_t)K, kh, K, eps, 1.0);
            oracle_l2norm(q + (t * Hk + j) * (int64_t)K, qh, K, eps, qscale);
            /* decay */
            for (size_t e = 0; e < (size_t)K * V; ++e)
                S[e] *= gamma;
            /* delta: u = beta * (v - S^T khat) */
            const double *vt = v + (t * Hv + h) * (int64_t)V;
            for (int c = 0; c < V; ++c) {
                double r = 0.0;
                for (int kk = 0; kk < K; ++kk)
                    r += S[(size_t)kk * V + c] * kh[kk];
                u[c] = beta * (vt[c] - r);
            }
            /* rank-1 update S += khat u^T */
            for (int kk = 0; kk < K; ++kk)
                for (int c = 0; c < V; ++c)
                    S[(size_t)kk * V + c] += kh[kk] * u[c];
            /* output o = S^T qhat */
            double *ot = out + (t * Hv + h) * (int64_t)V;
            for (int c = 0; c < V; ++c) {
                double o = 0.0;
                for (int kk = 0; kk < K; ++kk)
                    o += S[(size_t)kk * V + c] * qh[kk];
                ot[c] = o;
            }
            if (intermediate) {
                char *it = (char *)intermediate + ((size_t)t * Hv + h) * (size_t)K * V * esize;
                for (int kk = 0; kk < K; ++kk)
                    for (int c = 0; c < V; ++c)
                        tile_put(it, kk * row_stride + c * col_stride, S[(size_t)kk * V + c], bf16);
            }
        }
        if (!no_final_writeback)
            for (int kk = 0; kk < K; ++kk)
                for (int c = 0; c < V; ++c)
                    tile_put(tile, kk * row_stride + c * col_stride, S[(size_t)kk * V + c], bf16);
        free(S); free(kh); free(qh); free(u);
    }
    return status;
}

/*
 * The gating step on its own (the kernel the fused op absorbs):
 * g[t,h] = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h]), beta[t,h] =
 * sigmoid(b[t,h]); a, b, g, beta dense [N, Hv].
 */
int gdn_oracle_gating(const double *a, const double *b, const double *A_log,
                      const double *dt_bias, double *g, double *beta,
                      int64_t N, int Hv)
{
    if (N < 0 || Hv <= 0)
        return ORACLE_ERR_ARG;
    if (N > 0 && (!a || !b || !A_log || !dt_bias || !g || !beta))
        return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < N; ++t)
        for (int h = 0; h < Hv; ++h) {
            const int64_t e = t * Hv + h;
            g[e] = -exp(A_log[h]) * oracle_softplus(a[e] + dt_bias[h]);
            beta[e] = oracle_sigmoid(b[e]);
        }
    return ORACLE_OK;
}

int gdn_oracle_abi_version(void) { return 1; }
