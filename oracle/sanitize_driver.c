/*
 * Sanitizer driver for the CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Built together with oracle.c by tests/test_oracle_sanitized.py under gcc's
 * AddressSanitizer and UndefinedBehaviorSanitizer (host code only; nothing here
 * touches a GPU). Every oracle entry point runs on small, ragged shapes whose
 * buffers are heap blocks of exactly the documented sizes, so a read or write one
 * element past a tensor, a signed overflow in an index, or a misaligned access
 * aborts the run. It also checks that the sampled forms agree with the full forms
 * element for element, and that every result is finite. Exit status 0 means clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_conv_act_pool(const void* x, const void* w, const float* b, int dtype, int N, int Cin, int H, int W,
                         int Cout, int act, int pool, double* out);
int oracle_conv_pool_sample(const void* x, const void* w, const float* b, int dtype, int N, int Cin, int H, int W,
                            int Cout, int act, int count, const int* n_idx, const int* oc_idx, double* out);
int oracle_conv_point_sample(const void* x, const void* w, const float* b, int dtype, int N, int Cin, int H, int W,
                             int Cout, int act, int count, const int* n_idx, const int* oc_idx, const int* oh_idx,
                             const int* ow_idx, double* out);
int oracle_conv2d_act_pool(const void* x, const void* w, const float* b, int dtype, int N, int Cin, int H, int W,
                           int Cout, int K, int S, int P, int act, int pool, double* out);
int oracle_conv2d_pool_sample(const void* x, const void* w, const float* b, int dtype, int N, int Cin, int H, int W,
                              int Cout, int K, int S, int P, int act, int count, const int* n_idx, const int* oc_idx,
                              double* out);
int oracle_conv2d_point_sample(const void* x, const void* w, const float* b, int dtype, int N, int Cin, int H, int W,
                               int Cout, int K, int S, int P, int act, int count, const int* n_idx,
                               const int* oc_idx, const int* oh_idx, const int* ow_idx, double* out);
int oracle_gemm_lse_mish(const void* X, const void* Wt, const float* b, int dtype, int M, int K, int N, double scale,
                         double cmin, double cmax, int count, const int* rows, double* out, double* z_out);
int oracle_lse_mish_rows(const double* c, int M, int N, double* out, double* z_out);
int oracle_act_pool_map(const float* x, int N, int C, int H, int W, int act, double* out);
int oracle_act_elementwise(const float* x, long long count, int act, double* out);
int oracle_scale_clamp_lse_mish(const float* y, int M, int N, double scale, double cmin, double cmax, double* out,
                                double* z_out);

static uint64_t g_state = 0x243F6A8885A308D3ull;
static double next_unit(void) { /* a 64-bit LCG; its top 53 bits as a value in [-1, 1) */
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

/* a tensor of n elements, exactly n * size bytes (ASan guards both ends) */
static void* tensor(size_t n, int dtype, double scale) {
    if (dtype == 1) {
        uint16_t* t = (uint16_t*)malloc(n * sizeof(uint16_t));
        for (size_t i = 0; i < n; ++i) {
            float f = (float)(scale * next_unit());
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            t[i] = (uint16_t)(u >> 16);
        }
        return t;
    }
    float* t = (float*)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) t[i] = (float)(scale * next_unit());
    return t;
}

static int g_fail = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            g_fail = 1;                                   \
        }                                                 \
    } while (0)

static int all_finite(const double* v, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

/* conv with geometry (K, S, P); K == 3, S == 1, P == 0 also runs the 3x3 entry points */
static void run_conv(int dtype, int N, int Cin, int H, int W, int Cout, int K, int S, int P, int act) {
    const int OH = (H + 2 * P - K) / S + 1, OW = (W + 2 * P - K) / S + 1;
    void* x = tensor((size_t)N * Cin * H * W, dtype, 2.0);
    void* w = tensor((size_t)Cout * Cin * K * K, dtype, 0.5);
    float* b = (float*)tensor((size_t)Cout, 0, 0.1);
    double* pooled = (double*)malloc((size_t)N * Cout * sizeof(double));
    double* full = (double*)malloc((size_t)N * Cout * OH * OW * sizeof(double));
    CHECK(oracle_conv2d_act_pool(x, w, b, dtype, N, Cin, H, W, Cout, K, S, P, act, 1, pooled) == 0, "conv2d pool");
    CHECK(oracle_conv2d_act_pool(x, w, b, dtype, N, Cin, H, W, Cout, K, S, P, act, 0, full) == 0, "conv2d full");
    CHECK(all_finite(pooled, (size_t)N * Cout) && all_finite(full, (size_t)N * Cout * OH * OW), "finite");
    /* samples: every (n, oc) pair and the four corners of every map */
    const int np = N * Cout, nq = 4 * N * Cout;
    int* pn = (int*)malloc(np * sizeof(int));
    int* po = (int*)malloc(np * sizeof(int));
    int* qn = (int*)malloc(nq * sizeof(int));
    int* qo = (int*)malloc(nq * sizeof(int));
    int* qh = (int*)malloc(nq * sizeof(int));
    int* qw = (int*)malloc(nq * sizeof(int));
    double* ps = (double*)malloc(np * sizeof(double));
    double* qs = (double*)malloc(nq * sizeof(double));
    for (int i = 0; i < np; ++i) {
        pn[i] = i / Cout;
        po[i] = i % Cout;
        for (int c = 0; c < 4; ++c) {
            qn[4 * i + c] = pn[i];
            qo[4 * i + c] = po[i];
            qh[4 * i + c] = (c & 1) ? OH - 1 : 0;
            qw[4 * i + c] = (c & 2) ? OW - 1 : 0;
        }
    }
    CHECK(oracle_conv2d_pool_sample(x, w, b, dtype, N, Cin, H, W, Cout, K, S, P, act, np, pn, po, ps) == 0,
          "conv2d pool sample");
    CHECK(oracle_conv2d_point_sample(x, w, b, dtype, N, Cin, H, W, Cout, K, S, P, act, nq, qn, qo, qh, qw, qs) == 0,
          "conv2d point sample");
    for (int i = 0; i < np; ++i) CHECK(ps[i] == pooled[i], "pool sample %d", i);
    for (int i = 0; i < nq; ++i)
        CHECK(qs[i] == full[(((size_t)qn[i] * Cout + qo[i]) * OH + qh[i]) * OW + qw[i]], "point sample %d", i);
    if (K == 3 && S == 1 && P == 0) {
        double* p3 = (double*)malloc((size_t)N * Cout * sizeof(double));
        double* f3 = (double*)malloc((size_t)N * Cout * OH * OW * sizeof(double));
        CHECK(oracle_conv_act_pool(x, w, b, dtype, N, Cin, H, W, Cout, act, 1, p3) == 0, "conv pool");
        CHECK(oracle_conv_act_pool(x, w, b, dtype, N, Cin, H, W, Cout, act, 0, f3) == 0, "conv full");
        CHECK(oracle_conv_pool_sample(x, w, b, dtype, N, Cin, H, W, Cout, act, np, pn, po, ps) == 0, "conv sample");
        CHECK(oracle_conv_point_sample(x, w, b, dtype, N, Cin, H, W, Cout, act, nq, qn, qo, qh, qw, qs) == 0,
              "conv point sample");
        for (int i = 0; i < np; ++i) CHECK(p3[i] == pooled[i] && ps[i] == pooled[i], "3x3 pool %d", i);
        for (size_t i = 0; i < (size_t)N * Cout * OH * OW; ++i) CHECK(f3[i] == full[i], "3x3 full %zu", i);
        free(p3);
        free(f3);
    }
    free(x); free(w); free(b); free(pooled); free(full);
    free(pn); free(po); free(qn); free(qo); free(qh); free(qw); free(ps); free(qs);
}

static void run_gemm(int dtype, int M, int K, int N) {
    void* X = tensor((size_t)M * K, dtype, 1.0);
    void* Wt = tensor((size_t)N * K, dtype, 0.1);
    float* b = (float*)tensor((size_t)N, 0, 0.1);
    double* out = (double*)malloc((size_t)M * sizeof(double));
    double* z = (double*)malloc((size_t)M * sizeof(double));
    CHECK(oracle_gemm_lse_mish(X, Wt, b, dtype, M, K, N, 4.0, -10.0, 10.0, 0, NULL, out, z) == 0, "gemm");
    CHECK(all_finite(out, M) && all_finite(z, M), "gemm finite");
    int rows[3] = {M - 1, 0, M / 2};
    double o3[3], z3[3];
    CHECK(oracle_gemm_lse_mish(X, Wt, b, dtype, M, K, N, 4.0, -10.0, 10.0, 3, rows, o3, z3) == 0, "gemm rows");
    for (int i = 0; i < 3; ++i) CHECK(o3[i] == out[rows[i]] && z3[i] == z[rows[i]], "gemm row %d", rows[i]);
    free(X); free(Wt); free(b); free(out); free(z);
}

static void run_epilogues(int N, int C, int H, int W) {
    const size_t n = (size_t)N * C * H * W;
    float* x = (float*)tensor(n, 0, 4.0);
    double* pooled = (double*)malloc((size_t)N * C * sizeof(double));
    double* ew = (double*)malloc(n * sizeof(double));
    for (int act = 0; act < 4; ++act) {
        CHECK(oracle_act_pool_map(x, N, C, H, W, act, pooled) == 0, "act pool");
        CHECK(oracle_act_elementwise(x, (long long)n, act, ew) == 0, "act elementwise");
        CHECK(all_finite(pooled, (size_t)N * C) && all_finite(ew, n), "epilogue finite");
    }
    const int M = N * C, R = H * W;
    double* out = (double*)malloc((size_t)M * sizeof(double));
    double* z = (double*)malloc((size_t)M * sizeof(double));
    double* c = (double*)malloc(n * sizeof(double));
    CHECK(oracle_scale_clamp_lse_mish(x, M, R, 4.0, -10.0, 10.0, out, z) == 0, "scale clamp lse");
    for (size_t i = 0; i < n; ++i) c[i] = fmin(fmax(4.0 * (double)x[i], -10.0), 10.0);
    double* out2 = (double*)malloc((size_t)M * sizeof(double));
    CHECK(oracle_lse_mish_rows(c, M, R, out2, NULL) == 0, "lse rows");
    for (int m = 0; m < M; ++m) CHECK(out2[m] == out[m], "lse row %d", m);
    free(x); free(pooled); free(ew); free(out); free(z); free(c); free(out2);
}

int main(void) {
    static const int shapes[][5] = {  /* N, Cin, H, W, Cout: ragged, tiny, one past chunk and tile sizes */
        {1, 1, 3, 3, 1}, {2, 3, 7, 5, 2}, {1, 17, 6, 9, 3}, {2, 5, 11, 4, 7}, {1, 33, 5, 6, 2}};
    for (int s = 0; s < 5; ++s)
        for (int dtype = 0; dtype < 2; ++dtype)
            for (int act = 0; act < 4; ++act) {
                const int* sh = shapes[s];
                run_conv(dtype, sh[0], sh[1], sh[2], sh[3], sh[4], 3, 1, 0, act);
            }
    for (int K = 1; K <= 5; K += 2)
        for (int S = 1; S <= 2; ++S)
            for (int P = 0; P < K; ++P)
                for (int dtype = 0; dtype < 2; ++dtype) {
                    const int H = K > 2 * P ? K - 2 * P + 3 : 4, W = H + 2;
                    run_conv(dtype, 2, 5, H, W, 3, K, S, P, (K + S + P + dtype) % 4);
                }
    for (int dtype = 0; dtype < 2; ++dtype) {
        run_gemm(dtype, 1, 1, 1);
        run_gemm(dtype, 5, 17, 9);
        run_gemm(dtype, 3, 64, 130);
    }
    run_epilogues(2, 3, 5, 7);
    run_epilogues(1, 1, 1, 1);
    if (g_fail) return 1;
    printf("oracle sanitizer driver: clean\n");
    return 0;
}
