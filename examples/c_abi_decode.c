/*
 * libgdn from plain C: one decode step through the C-ABI, with buffers from
 * the HIP runtime and no Python or PyTorch.  It runs two calls and checks
 * each against a closed form of the gated delta rule (vLLM PR #35777,
 * implementation section: the gating folded into the recurrent update):
 *
 *  1. From a zero state, with l2norm_eps = 0, the update leaves
 *     S = beta * khat v^T and returns out = beta * (khat . qhat) * v.
 *  2. With g = 0 (A_log = -1000), beta = 1 (b = +1000) and q = k, one more
 *     update makes S^T khat = v exactly, so out = K^-1/2 * v.
 *
 * A padded sequence (slot -1) must leave its output rows alone, and slots no
 * sequence names must keep their bytes.  Exits 0 and prints "ok" on success.
 *
 * Build (done by the package build): gcc -std=c11 -D__HIP_PLATFORM_AMD__
 *   -I include -I /opt/rocm/include examples/c_abi_decode.c -L <libdir> -lgdn
 *   -L /opt/rocm/lib -lamdhip64 -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

enum { B = 4, HK = 2, HV = 4, K = 128, V = 128, SLOTS = 6, N = B };
static const int32_t kSlots[B] = {3, -1, 0, 5};   /* sequence 1 is padding */
static const float kSentinel = 12345.0f;

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(2);                                                               \
        }                                                                          \
    } while (0)

#define GDN_OK_OR_DIE(x)                                                            \
    do {                                                                            \
        gdn_status s_ = (x);                                                        \
        if (s_ != GDN_OK) {                                                         \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__,                  \
                    gdn_status_string(s_), gdn_last_error_message());              \
            exit(2);                                                                \
        }                                                                           \
    } while (0)

/* Deterministic values in [-1, 1). */
static uint32_t g_seed = 12345u;
static float next_value(void) {
    g_seed = g_seed * 1664525u + 1013904223u;
    return (float)((g_seed >> 8) & 0xFFFFFF) / 8388608.0f - 1.0f;
}

static void fill(float* x, size_t n) {
    for (size_t i = 0; i < n; ++i) x[i] = next_value();
}

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static double norm(const float* x, int n) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += (double)x[i] * x[i];
    return sqrt(s);
}

static int failures = 0;
static void check(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

int main(void) {
    const size_t n_qk = (size_t)N * HK * K, n_v = (size_t)N * HV * V, n_ab = (size_t)N * HV;
    const size_t n_tile = (size_t)K * V, n_pool = (size_t)SLOTS * HV * n_tile;
    float *q = malloc(n_qk * 4), *k = malloc(n_qk * 4), *v = malloc(n_v * 4);
    float *a = malloc(n_ab * 4), *b = malloc(n_ab * 4), *out = malloc(n_v * 4);
    float *pool0 = calloc(n_pool, 4), *pool = malloc(n_pool * 4);
    float A_log[HV], dt_bias[HV];
    if (!q || !k || !v || !a || !b || !out || !pool0 || !pool) return 2;

    fill(q, n_qk);
    fill(k, n_qk);
    fill(v, n_v);
    fill(a, n_ab);
    fill(b, n_ab);
    for (int h = 0; h < HV; ++h) {
        A_log[h] = logf(1.0f + 3.0f * (float)h);
        dt_bias[h] = 0.25f * next_value();
    }
    /* live slots start at zero; the others hold a pattern that must survive */
    for (int s = 0; s < SLOTS; ++s) {
        int named = 0;
        for (int i = 0; i < B; ++i) named |= kSlots[i] == s;
        if (!named) fill(pool0 + (size_t)s * HV * n_tile, (size_t)HV * n_tile);
    }
    for (size_t i = 0; i < n_v; ++i) out[i] = kSentinel;

    float* d_q = to_device(q, n_qk * 4);
    float* d_k = to_device(k, n_qk * 4);
    float* d_v = to_device(v, n_v * 4);
    float* d_a = to_device(a, n_ab * 4);
    float* d_b = to_device(b, n_ab * 4);
    float* d_A = to_device(A_log, sizeof A_log);
    float* d_dt = to_device(dt_bias, sizeof dt_bias);
    float* d_pool = to_device(pool0, n_pool * 4);
    int32_t* d_idx = to_device(kSlots, sizeof kSlots);
    float* d_out = to_device(out, n_v * 4);

    gdn_config cfg;
    gdn_default_config(&cfg);
    cfg.num_seqs = B;
    cfg.tokens_per_seq = 1;
    cfg.num_tokens = N;
    cfg.num_k_heads = HK;
    cfg.num_v_heads = HV;
    cfg.head_k_dim = K;
    cfg.head_v_dim = V;
    cfg.num_slots = SLOTS;
    cfg.act_dtype = GDN_DTYPE_F32;
    cfg.l2norm_eps = 0.0f;

    printf("libgdn ABI version %d\n", gdn_abi_version());
    gdn_launch_info info;
    GDN_OK_OR_DIE(gdn_plan(&cfg, 0, 0, &info));
    printf("plan: kernel family %d, %lld workgroups of %d threads, %d bytes of LDS\n",
           info.kernel_family, (long long)info.workgroups, info.threads_per_group, info.lds_bytes);

    /* an unsupported head size is refused before anything is launched */
    gdn_config bad = cfg;
    bad.head_k_dim = 48;
    check(gdn_validate(d_q, d_k, d_v, d_a, d_b, d_A, d_dt, d_pool, d_idx, NULL, d_out, NULL, &bad) ==
              GDN_ERR_UNSUPPORTED_SHAPE,
          "K = 48 must be rejected");
    printf("K = 48 rejected: %s\n", gdn_last_error_message());

    /* ---- call 1: zero state */
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    GDN_OK_OR_DIE(gdn_gating_delta_rule_update(d_q, d_k, d_v, d_a, d_b, d_A, d_dt, d_pool, d_idx,
                                               NULL, d_out, NULL, &cfg, stream));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(out, d_out, n_v * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(pool, d_pool, n_pool * 4, hipMemcpyDeviceToHost));

    const double scale = 1.0 / sqrt((double)K);
    double err = 0.0, ref_max = 0.0, serr = 0.0, sref_max = 0.0;
    for (int i = 0; i < B; ++i) {
        for (int h = 0; h < HV; ++h) {
            const int j = h / (HV / HK);
            const float* qi = q + ((size_t)i * HK + j) * K;
            const float* ki = k + ((size_t)i * HK + j) * K;
            const float* vi = v + ((size_t)i * HV + h) * V;
            const float* oi = out + ((size_t)i * HV + h) * V;
            if (kSlots[i] < 0) {
                for (int c = 0; c < V; ++c) check(oi[c] == kSentinel, "padded output row written");
                continue;
            }
            const double nq = norm(qi, K), nk = norm(ki, K);
            double kq = 0.0;
            for (int r = 0; r < K; ++r) kq += (ki[r] / nk) * (scale * qi[r] / nq);
            const double beta = 1.0 / (1.0 + exp(-(double)b[(size_t)i * HV + h]));
            const float* S = pool + ((size_t)kSlots[i] * HV + h) * n_tile;
            for (int c = 0; c < V; ++c) {
                const double ref = beta * kq * vi[c];
                err = fmax(err, fabs(oi[c] - ref));
                ref_max = fmax(ref_max, fabs(ref));
            }
            for (int r = 0; r < K; ++r)
                for (int c = 0; c < V; ++c) {
                    const double ref = beta * (ki[r] / nk) * vi[c];
                    serr = fmax(serr, fabs(S[(size_t)r * V + c] - ref));
                    sref_max = fmax(sref_max, fabs(ref));
                }
        }
    }
    printf("call 1: max |out - beta (khat.qhat) v| / max|ref| = %.2e, state %.2e\n",
           err / ref_max, serr / sref_max);
    check(err <= 1e-5 * ref_max, "call 1 output");
    check(serr <= 1e-5 * sref_max, "call 1 state");
    for (int s = 0; s < SLOTS; ++s) {
        int named = 0;
        for (int i = 0; i < B; ++i) named |= kSlots[i] == s && kSlots[i] >= 0;
        if (!named)
            check(memcmp(pool + (size_t)s * HV * n_tile, pool0 + (size_t)s * HV * n_tile,
                         (size_t)HV * n_tile * 4) == 0,
                  "a slot outside the batch changed");
    }

    /* ---- call 2: g = 0, beta = 1, q = k on the state call 1 left */
    for (int h = 0; h < HV; ++h) A_log[h] = -1000.0f;
    for (size_t i = 0; i < n_ab; ++i) b[i] = 1000.0f;
    fill(v, n_v);
    HIP_OK(hipMemcpy(d_A, A_log, sizeof A_log, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_b, b, n_ab * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, v, n_v * 4, hipMemcpyHostToDevice));
    GDN_OK_OR_DIE(gdn_gating_delta_rule_update(d_k, d_k, d_v, d_a, d_b, d_A, d_dt, d_pool, d_idx,
                                               NULL, d_out, NULL, &cfg, stream));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(out, d_out, n_v * 4, hipMemcpyDeviceToHost));
    err = 0.0;
    ref_max = 0.0;
    for (int i = 0; i < B; ++i) {
        for (int h = 0; h < HV; ++h) {
            const float* oi = out + ((size_t)i * HV + h) * V;
            const float* vi = v + ((size_t)i * HV + h) * V;
            for (int c = 0; c < V; ++c) {
                if (kSlots[i] < 0) {
                    check(oi[c] == kSentinel, "padded output row written");
                    continue;
                }
                err = fmax(err, fabs(oi[c] - scale * vi[c]));
                ref_max = fmax(ref_max, fabs(scale * vi[c]));
            }
        }
    }
    printf("call 2: max |out - K^-1/2 v| / max|ref| = %.2e\n", err / ref_max);
    check(err <= 1e-5 * ref_max, "call 2 output");

    HIP_OK(hipStreamDestroy(stream));
    hipFree(d_q); hipFree(d_k); hipFree(d_v); hipFree(d_a); hipFree(d_b); hipFree(d_A);
    hipFree(d_dt); hipFree(d_pool); hipFree(d_idx); hipFree(d_out);
    free(q); free(k); free(v); free(a); free(b); free(out); free(pool0); free(pool);
    if (failures) {
        printf("%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
