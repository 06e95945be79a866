/*
 * CPU oracle for the fused conv / GEMM epilogues -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct fp64 implementation of what the hot path
 * computes. It is used by the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark; nothing on the product path may call it. It shares no
 * code with the HIP library: its own loops, double precision throughout, libm
 * erf / exp / log1p / tanh / log.
 *
 * Sources (the three POPCORNBENCH level-2 pages, Kimi-K2.6 traces):
 *  - "Kimi-K2.6 l2_p4" (Conv2d -> Mish -> Mish): the direct-convolution sum
 *    with bias over in-channels and the 3x3 window, valid padding, output
 *    size H-2; Mish = x * tanh(softplus(x)) applied twice.
 *  - "Kimi-K2.6 l2_p67" (Conv2d -> GELU -> AdaptiveAvgPool2d(1)): the exact
 *    erf form of GELU (PyTorch's approximate='none'), then the mean of each
 *    (n, c) feature map over the valid output positions. The same page also
 *    writes the tanh approximation of GELU (PyTorch's approximate='tanh'),
 *    offered here as a separate activation.
 *  - "Kimi-K2.6 l2_p22" (Linear -> scale -> x+x -> clamp -> logsumexp ->
 *    x*mish(x)): y = x W^T + b, scaled (the page's x2 then x+x is x4),
 *    clamped, the max-shifted logsumexp per row, then z * mish(z).
 *
 * Layouts: x NCHW contiguous, w OIHW contiguous, b [Cout]; GEMM X [M][K],
 * W [N][K] (nn.Linear), b [N]. x and w are float32, or bfloat16 bit patterns
 * (dtype = 1) that are widened exactly to double.
 *
 * Parity pins for every function here live in tests/test_oracle.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_GELU 1
#define ORACLE_ACT_MISH2 2
#define ORACLE_ACT_GELU_TANH 3

static double widen_bf16(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void* p, size_t i, int dtype) {
    if (dtype == 1) return widen_bf16(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

/* softplus(v) = log(1 + e^v) in the overflow-free form max(v,0) + log1p(e^-|v|)
 * (the stable softplus discussed on the l2_p22 and l2_p4 pages). */
double oracle_softplus(double v) {
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

/* Mish(v) = v * tanh(softplus(v)) (l2_p4 page, definition of Mish). */
double oracle_mish(double v) {
    return v * tanh(oracle_softplus(v));
}

/* GELU(v) = 0.5 v (1 + erf(v / sqrt 2)), the exact form (l2_p67 page). */
double oracle_gelu(double v) {
    return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
}

/* Tanh approximation of GELU (l2_p67 page, where it weighs the tanh form against
 * the exact one): 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))). */
double oracle_gelu_tanh(double v) {
    const double k = sqrt(2.0 / 3.14159265358979323846); /* sqrt(2 / pi) */
    return 0.5 * v * (1.0 + tanh(k * (v + 0.044715 * v * v * v)));
}

/* Pointwise activation: 0 none, 1 exact GELU, 2 Mish applied twice, 3 tanh GELU. */
double oracle_act(double v, int act) {
    switch (act) {
        case ORACLE_ACT_GELU: return oracle_gelu(v);
        case ORACLE_ACT_MISH2: return oracle_mish(oracle_mish(v));
        case ORACLE_ACT_GELU_TANH: return oracle_gelu_tanh(v);
        default: return v;
    }
}

/* One pre-activation value: b[oc] + sum_{ic,kh,kw} w[oc,ic,kh,kw] x[n,ic,oh+kh,ow+kw]
 * (cross-correlation, no kernel flip, stride 1, no padding). */
static double conv_pre(const void* x, const void* w, const float* b, int dtype,
                       int Cin, int H, int W, int n, int oc, int oh, int ow) {
    double acc = 0.0;
    for (int ic = 0; ic < Cin; ++ic) {
        for (int kh = 0; kh < 3; ++kh) {
            for (int kw = 0; kw < 3; ++kw) {
                size_t xi = (((size_t)n * Cin + ic) * H + (oh + kh)) * W + (ow + kw);
                size_t wi = (((size_t)oc * Cin + ic) * 3 + kh) * 3 + kw;
                acc += load_elem(w, wi, dtype) * load_elem(x, xi, dtype);
            }
        }
    }
    return acc + (double)b[oc];
}

/* Mean over the valid OHxOW map of act(pre[n,oc,.,.]). */
static double conv_pool_one(const void* x, const void* w, const float* b, int dtype,
                            int Cin, int H, int W, int n, int oc, int act) {
    int OH = H - 2, OW = W - 2;
    double s = 0.0;
    for (int oh = 0; oh < OH; ++oh)
        for (int ow = 0; ow < OW; ++ow)
            s += oracle_act(conv_pre(x, w, b, dtype, Cin, H, W, n, oc, oh, ow), act);
    return s / ((double)OH * (double)OW);
}

/*
 * Full fused conv: out is [N][Cout] (pool = 1) or [N][Cout][H-2][W-2] (pool = 0),
 * all in double. Returns 0, or -1 on a bad argument.
 */
int oracle_conv_act_pool(const void* x, const void* w, const float* b, int dtype,
                         int N, int Cin, int H, int W, int Cout, int act, int pool,
                         double* out) {
    if (!x || !w || !b || !out || N <= 0 || Cin <= 0 || H < 3 || W < 3 || Cout <= 0) return -1;
    int OH = H - 2, OW = W - 2;
    long long NC = (long long)N * Cout;
    if (pool) {
#pragma omp parallel for schedule(dynamic)
        for (long long t = 0; t < NC; ++t) {
            int n = (int)(t / Cout), oc = (int)(t % Cout);
            out[t] = conv_pool_one(x, w, b, dtype, Cin, H, W, n, oc, act);
        }
    } else {
        long long rows = NC * OH;
#pragma omp parallel for schedule(dynamic, 16)
        for (long long t = 0; t < rows; ++t) {
            int oh = (int)(t % OH);
            long long nc = t / OH;
            int n = (int)(nc / Cout), oc = (int)(nc % Cout);
            double* o = out + (size_t)t * OW;
            for (int ow = 0; ow < OW; ++ow)
                o[ow] = oracle_act(conv_pre(x, w, b, dtype, Cin, H, W, n, oc, oh, ow), act);
        }
    }
    return 0;
}

/* Pooled outputs for `count` selected (n, oc) pairs. */
int oracle_conv_pool_sample(const void* x, const void* w, const float* b, int dtype,
                            int N, int Cin, int H, int W, int Cout, int act,
                            int count, const int* n_idx, const int* oc_idx, double* out) {
    if (!x || !w || !b || !out || H < 3 || W < 3) return -1;
    for (int i = 0; i < count; ++i)
        if (n_idx[i] < 0 || n_idx[i] >= N || oc_idx[i] < 0 || oc_idx[i] >= Cout) return -1;
#pragma omp parallel for schedule(dynamic)
    for (int i = 0; i < count; ++i)
        out[i] = conv_pool_one(x, w, b, dtype, Cin, H, W, n_idx[i], oc_idx[i], act);
    return 0;
}

/* Activated outputs act(pre[n,oc,oh,ow]) at `count` selected points. */
int oracle_conv_point_sample(const void* x, const void* w, const float* b, int dtype,
                             int N, int Cin, int H, int W, int Cout, int act,
                             int count, const int* n_idx, const int* oc_idx,
                             const int* oh_idx, const int* ow_idx, double* out) {
    if (!x || !w || !b || !out || H < 3 || W < 3) return -1;
    for (int i = 0; i < count; ++i)
        if (n_idx[i] < 0 || n_idx[i] >= N || oc_idx[i] < 0 || oc_idx[i] >= Cout ||
            oh_idx[i] < 0 || oh_idx[i] >= H - 2 || ow_idx[i] < 0 || ow_idx[i] >= W - 2) return -1;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < count; ++i)
        out[i] = oracle_act(conv_pre(x, w, b, dtype, Cin, H, W, n_idx[i], oc_idx[i],
                                     oh_idx[i], ow_idx[i]), act);
    return 0;
}

/* ---------------------------------------------------------------------------------
 * General geometry: a square K x K kernel, stride S, zero padding P on all four sides
 * (nn.Conv2d's kernel_size / stride / padding). The pages fix K = 3, S = 1, P = 0; the
 * same direct sum with those three parameters opened up:
 *   pre[n,oc,oh,ow] = b[oc] + sum_{ic,kh,kw} w[oc,ic,kh,kw] * xp[n,ic,oh*S+kh-P,ow*S+kw-P]
 * where xp reads zero outside 0 <= row < H, 0 <= col < W, and
 *   OH = (H + 2P - K) / S + 1,  OW = (W + 2P - K) / S + 1   (integer division).
 * --------------------------------------------------------------------------------- */
static double conv2d_pre(const void* x, const void* w, const float* b, int dtype, int Cin, int H, int W,
                         int K, int S, int P, int n, int oc, int oh, int ow) {
    double acc = 0.0;
    for (int ic = 0; ic < Cin; ++ic) {
        for (int kh = 0; kh < K; ++kh) {
            int ih = oh * S + kh - P;
            if (ih < 0 || ih >= H) continue; /* zero padding */
            for (int kw = 0; kw < K; ++kw) {
                int iw = ow * S + kw - P;
                if (iw < 0 || iw >= W) continue;
                size_t xi = (((size_t)n * Cin + ic) * H + ih) * W + iw;
                size_t wi = (((size_t)oc * Cin + ic) * K + kh) * K + kw;
                acc += load_elem(w, wi, dtype) * load_elem(x, xi, dtype);
            }
        }
    }
    return acc + (double)b[oc];
}

static int conv2d_geometry(int H, int W, int K, int S, int P, int* OH, int* OW) {
    if (K < 1 || S < 1 || P < 0 || H + 2 * P < K || W + 2 * P < K) return -1;
    *OH = (H + 2 * P - K) / S + 1;
    *OW = (W + 2 * P - K) / S + 1;
    return 0;
}

/* Mean over the OH x OW output map of act(pre[n,oc,.,.]). */
static double conv2d_pool_one(const void* x, const void* w, const float* b, int dtype, int Cin, int H, int W,
                              int K, int S, int P, int n, int oc, int act) {
    int OH = 0, OW = 0;
    conv2d_geometry(H, W, K, S, P, &OH, &OW); /* validated by every caller */
    double s = 0.0;
    for (int oh = 0; oh < OH; ++oh)
        for (int ow = 0; ow < OW; ++ow)
            s += oracle_act(conv2d_pre(x, w, b, dtype, Cin, H, W, K, S, P, n, oc, oh, ow), act);
    return s / ((double)OH * (double)OW);
}

/* Full general-geometry conv: out [N][Cout] (pool = 1) or [N][Cout][OH][OW] (pool = 0). */
int oracle_conv2d_act_pool(const void* x, const void* w, const float* b, int dtype,
                           int N, int Cin, int H, int W, int Cout, int K, int S, int P,
                           int act, int pool, double* out) {
    int OH, OW;
    if (!x || !w || !b || !out || N <= 0 || Cin <= 0 || Cout <= 0 || H <= 0 || W <= 0) return -1;
    if (conv2d_geometry(H, W, K, S, P, &OH, &OW)) return -1;
    long long NC = (long long)N * Cout;
    if (pool) {
#pragma omp parallel for schedule(dynamic)
        for (long long t = 0; t < NC; ++t)
            out[t] = conv2d_pool_one(x, w, b, dtype, Cin, H, W, K, S, P, (int)(t / Cout), (int)(t % Cout), act);
    } else {
        long long rows = NC * OH;
#pragma omp parallel for schedule(dynamic, 16)
        for (long long t = 0; t < rows; ++t) {
            int oh = (int)(t % OH);
            long long nc = t / OH;
            int n = (int)(nc / Cout), oc = (int)(nc % Cout);
            double* o = out + (size_t)t * OW;
            for (int ow = 0; ow < OW; ++ow)
                o[ow] = oracle_act(conv2d_pre(x, w, b, dtype, Cin, H, W, K, S, P, n, oc, oh, ow), act);
        }
    }
    return 0;
}

/* Pooled general-geometry outputs for `count` selected (n, oc) pairs. */
int oracle_conv2d_pool_sample(const void* x, const void* w, const float* b, int dtype,
                              int N, int Cin, int H, int W, int Cout, int K, int S, int P, int act,
                              int count, const int* n_idx, const int* oc_idx, double* out) {
    int OH, OW;
    if (!x || !w || !b || !out || conv2d_geometry(H, W, K, S, P, &OH, &OW)) return -1;
    for (int i = 0; i < count; ++i)
        if (n_idx[i] < 0 || n_idx[i] >= N || oc_idx[i] < 0 || oc_idx[i] >= Cout) return -1;
#pragma omp parallel for schedule(dynamic)
    for (int i = 0; i < count; ++i)
        out[i] = conv2d_pool_one(x, w, b, dtype, Cin, H, W, K, S, P, n_idx[i], oc_idx[i], act);
    return 0;
}

/* Activated general-geometry outputs at `count` selected (n, oc, oh, ow) points. */
int oracle_conv2d_point_sample(const void* x, const void* w, const float* b, int dtype,
                               int N, int Cin, int H, int W, int Cout, int K, int S, int P, int act,
                               int count, const int* n_idx, const int* oc_idx,
                               const int* oh_idx, const int* ow_idx, double* out) {
    int OH, OW;
    if (!x || !w || !b || !out || conv2d_geometry(H, W, K, S, P, &OH, &OW)) return -1;
    for (int i = 0; i < count; ++i)
        if (n_idx[i] < 0 || n_idx[i] >= N || oc_idx[i] < 0 || oc_idx[i] >= Cout ||
            oh_idx[i] < 0 || oh_idx[i] >= OH || ow_idx[i] < 0 || ow_idx[i] >= OW) return -1;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < count; ++i)
        out[i] = oracle_act(conv2d_pre(x, w, b, dtype, Cin, H, W, K, S, P, n_idx[i], oc_idx[i],
                                       oh_idx[i], ow_idx[i]), act);
    return 0;
}

/*
 * GEMM + logsumexp + z*mish(z) for `count` selected rows (rows == NULL: all M rows).
 *   y[m,j] = scale * (sum_k X[m,k] W[j,k] + b[j]);  c = min(max(y, cmin), cmax)
 *   z[m]   = Mx + log(sum_j exp(c[m,j] - Mx)),   Mx = max_j c[m,j]
 *   out[m] = z * mish(z)
 * (l2_p22 page: the model's chain, and the two-pass max-shifted logsumexp.)
 * out[i] and (if non-NULL) z_out[i] receive row rows[i]'s results.
 */
int oracle_gemm_lse_mish(const void* X, const void* Wt, const float* b, int dtype,
                         int M, int K, int N, double scale, double cmin, double cmax,
                         int count, const int* rows, double* out, double* z_out) {
    if (!X || !Wt || !b || !out || M <= 0 || K <= 0 || N <= 0 || cmin > cmax) return -1;
    if (dtype != 0 && dtype != 1) return -1;
    int nrows = rows ? count : M;
    if (rows)
        for (int i = 0; i < count; ++i)
            if (rows[i] < 0 || rows[i] >= M) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic)
    for (int i = 0; i < nrows; ++i) {
        int m = rows ? rows[i] : i;
        double* c = (double*)malloc((size_t)N * sizeof(double));
        if (!c) { bad = 1; continue; }
        /* the scaled, clamped row and its maximum */
        double mx = -INFINITY;
        for (int j = 0; j < N; ++j) {
            double dot = 0.0;
            for (int k = 0; k < K; ++k)
                dot += load_elem(X, (size_t)m * K + k, dtype) * load_elem(Wt, (size_t)j * K + k, dtype);
            c[j] = fmin(fmax(scale * (dot + (double)b[j]), cmin), cmax);
            if (c[j] > mx) mx = c[j];
        }
        /* sum of exp(c - max), then the shifted log */
        double s = 0.0;
        for (int j = 0; j < N; ++j) s += exp(c[j] - mx);
        double z = mx + log(s);
        out[i] = z * oracle_mish(z);
        if (z_out) z_out[i] = z;
        free(c);
    }
    return bad ? -2 : 0;
}

/* Logsumexp + z*mish(z) of a given row-major [M][N] matrix of already-clamped values. */
int oracle_lse_mish_rows(const double* c, int M, int N, double* out, double* z_out) {
    if (!c || !out || M <= 0 || N <= 0) return -1;
    for (int m = 0; m < M; ++m) {
        const double* r = c + (size_t)m * N;
        double mx = -INFINITY;
        for (int j = 0; j < N; ++j) if (r[j] > mx) mx = r[j];
        double s = 0.0;
        for (int j = 0; j < N; ++j) s += exp(r[j] - mx);
        double z = mx + log(s);
        out[m] = z * oracle_mish(z);
        if (z_out) z_out[m] = z;
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------
 * Epilogue-only operations: the pages' own kernels that run after a separate
 * convolution or GEMM ("Kimi-K2.6 l2_p67": GELU + average pool over the conv output;
 * "Kimi-K2.6 l2_p4": Mish applied twice, elementwise, over the conv output;
 * "Kimi-K2.6 l2_p22": scale, clamp, row logsumexp and x*mish(x) over the Linear output).
 * --------------------------------------------------------------------------------- */

/* mean over count values of act(v[i]) */
double oracle_act_mean(const float* v, long long count, int act) {
    double s = 0.0;
    for (long long i = 0; i < count; ++i) s += oracle_act((double)v[i], act);
    return s / (double)count;
}

/* out[n][c] = mean over the H x W map of act(x[n][c][.][.]) */
int oracle_act_pool_map(const float* x, int N, int C, int H, int W, int act, double* out) {
    if (!x || !out || N <= 0 || C <= 0 || H <= 0 || W <= 0) return -1;
    long long planes = (long long)N * C, hw = (long long)H * W;
#pragma omp parallel for schedule(dynamic)
    for (long long p = 0; p < planes; ++p) out[p] = oracle_act_mean(x + p * hw, hw, act);
    return 0;
}

/* out[i] = act(x[i]) */
int oracle_act_elementwise(const float* x, long long count, int act, double* out) {
    if (!x || !out || count < 0) return -1;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < count; ++i) out[i] = oracle_act((double)x[i], act);
    return 0;
}

/* For each row of a given [M][N] matrix y: c = min(max(scale * y, cmin), cmax),
 * z = max-shifted logsumexp of the row, out = z * mish(z). */
int oracle_scale_clamp_lse_mish(const float* y, int M, int N, double scale, double cmin, double cmax,
                                double* out, double* z_out) {
    if (!y || !out || M <= 0 || N <= 0 || cmin > cmax) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic)
    for (int m = 0; m < M; ++m) {
        const float* r = y + (size_t)m * N;
        double* c = (double*)malloc((size_t)N * sizeof(double));
        if (!c) { bad = 1; continue; }
        double mx = -INFINITY;
        for (int j = 0; j < N; ++j) {
            c[j] = fmin(fmax(scale * (double)r[j], cmin), cmax);
            if (c[j] > mx) mx = c[j];
        }
        double s = 0.0;
        for (int j = 0; j < N; ++j) s += exp(c[j] - mx);
        double z = mx + log(s);
        out[m] = z * oracle_mish(z);
        if (z_out) z_out[m] = z;
        free(c);
    }
    return bad ? -2 : 0;
}
