/* Runs every entry of the CPU oracle (oracle/oracle.c) on small inputs, for a
 * build with the address and undefined-behaviour sanitizers: the router (both
 * kinds, k = E included), the permutation, the FFN in every weight format and
 * both activations, the combine, the whole layer with and without a shared
 * expert, the coverage set and both quantizers.  Inputs come from a local
 * splitmix64 stream.  Beyond memory safety it checks two invariants that need
 * no reference: the routing weights sum to the scale, and the permutation is
 * a bijection.  Prints one summary line; exit status 0 iff nothing failed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t g_state = 0x5A17u;
static double unif(void) {
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static float* fvec(size_t n, double lo, double hi) {
    float* v = malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) v[i] = (float)(lo + (hi - lo) * unif());
    return v;
}
static int8_t* codes(size_t n, int lo, int hi) {
    int8_t* v = malloc(n);
    for (size_t i = 0; i < n; ++i) v[i] = (int8_t)(lo + (int)((hi - lo + 1) * unif()));
    return v;
}

static int g_fail = 0;

static void experts_of(int fmt, int E, int d, int I, int act, oracle_experts* W) {
    W->fmt = fmt; W->E = E; W->d = d; W->inter = I; W->act = act;
    const size_t ngu = (size_t)E * 2 * I * d, ndn = (size_t)E * d * I;
    if (fmt == ORACLE_W_FP32) {
        W->gu = fvec(ngu, -0.1, 0.1); W->dn = fvec(ndn, -0.1, 0.1);
        W->gu_s = NULL; W->dn_s = NULL;
        return;
    }
    const int B = fmt == ORACLE_W_INT4_B128 ? 128 : 32;
    W->gu = fmt == ORACLE_W_INT8_ROW ? codes(ngu, -127, 127) : codes(ngu, -8, 7);
    W->dn = fmt == ORACLE_W_INT8_ROW ? codes(ndn, -127, 127) : codes(ndn, -8, 7);
    const size_t sgu = fmt == ORACLE_W_INT8_ROW ? (size_t)E * 2 * I : (size_t)E * 2 * I * (d / B);
    const size_t sdn = fmt == ORACLE_W_INT8_ROW ? (size_t)E * d : (size_t)E * d * (I / B);
    float* a = fvec(sgu, 1e-4, 2e-3);
    float* b = fvec(sdn, 1e-4, 2e-3);
    a[0] = 0.0f;  /* the int4 floor (and an int8 zero row) */
    b[0] = 1e-40f;
    W->gu_s = a; W->dn_s = b;
}
static void free_experts(oracle_experts* W) {
    free((void*)W->gu); free((void*)W->dn); free((void*)W->gu_s); free((void*)W->dn_s);
}

static void layer_case(int router, int fmt, int act, int E, int k, int d, int I, int T,
                       int shared) {
    oracle_layer_args L;
    memset(&L, 0, sizeof L);
    L.router = router;
    L.k = k;
    L.scale = router == ORACLE_ROUTER_SIGMOID_BIAS ? 2.446f : 1.0f;
    L.wr = fvec((size_t)E * d, -0.05, 0.05);
    L.bias = router == ORACLE_ROUTER_SIGMOID_BIAS ? fvec(E, -0.1, 0.1) : NULL;
    experts_of(fmt, E, d, I, act, &L.experts);
    L.has_shared = shared;
    if (shared) experts_of(ORACLE_W_FP32, 1, d, I, act, &L.shared);
    float* x = fvec((size_t)T * d, -2, 2);
    int32_t* idx = malloc((size_t)T * k * sizeof(int32_t));
    double* w = malloc((size_t)T * k * sizeof(double));
    double* gap = malloc((size_t)T * sizeof(double));
    double* y = malloc((size_t)T * d * sizeof(double));
    if (oracle_layer(&L, x, T, idx, w, gap, y) != 0) ++g_fail;
    for (int t = 0; t < T; ++t) {
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += w[(size_t)t * k + j];
        if (fabs(s - L.scale) > 1e-6 * L.scale) ++g_fail;
    }
    /* the separate steps on the same inputs */
    double* lg = malloc((size_t)T * E * sizeof(double));
    if (oracle_route(router, x, L.wr, L.bias, T, d, E, k, L.scale, idx, w, gap, lg) != 0) ++g_fail;
    int32_t* off = malloc((size_t)(E + 1) * sizeof(int32_t));
    int32_t* rt = malloc((size_t)T * k * sizeof(int32_t));
    int32_t* tr = malloc((size_t)T * k * sizeof(int32_t));
    if (oracle_permute(idx, T, k, E, off, rt, tr) != 0) ++g_fail;
    unsigned char* seen = calloc((size_t)T * k, 1);
    for (int q = 0; q < T * k; ++q) {
        if (tr[q] < 0 || tr[q] >= T * k || seen[tr[q]]) { ++g_fail; continue; }
        seen[tr[q]] = 1;
    }
    double* rows = malloc((size_t)T * k * d * sizeof(double));
    if (oracle_expert_rows(&L.experts, x, rt, off, rows) != 0) ++g_fail;
    float* rowsf = malloc((size_t)T * k * d * sizeof(float));
    for (size_t i = 0; i < (size_t)T * k * d; ++i) rowsf[i] = (float)rows[i];
    float* wf = malloc((size_t)T * k * sizeof(float));
    for (int i = 0; i < T * k; ++i) wf[i] = (float)w[i];
    oracle_combine(rowsf, tr, wf, NULL, x, T, k, d, y);
    double* h = malloc((size_t)I * sizeof(double));
    oracle_ffn(&L.experts, E - 1, x, y, h);
    free(h); free(wf); free(rowsf); free(rows); free(seen); free(tr); free(rt); free(off);
    free(lg); free(y); free(gap); free(w); free(idx); free(x);
    free_experts(&L.experts);
    if (shared) free_experts(&L.shared);
    free((void*)L.wr); free((void*)L.bias);
}

int main(void) {
    layer_case(ORACLE_ROUTER_SIGMOID_BIAS, ORACLE_W_INT8_ROW, ORACLE_ACT_SILU, 16, 4, 128, 64, 7, 1);
    layer_case(ORACLE_ROUTER_SOFTMAX, ORACLE_W_INT4_B32, ORACLE_ACT_SILU, 12, 8, 128, 64, 5, 0);
    layer_case(ORACLE_ROUTER_SOFTMAX, ORACLE_W_INT4_B128, ORACLE_ACT_GELU_TANH, 8, 2, 256, 128, 3, 0);
    layer_case(ORACLE_ROUTER_SIGMOID_BIAS, ORACLE_W_FP32, ORACLE_ACT_GELU_TANH, 8, 8, 64, 32, 2, 1);
    layer_case(ORACLE_ROUTER_SIGMOID_BIAS, ORACLE_W_INT8_ROW, ORACLE_ACT_SILU, 5, 5, 64, 32, 1, 0);

    uint64_t counts[40];
    for (int e = 0; e < 40; ++e) counts[e] = (uint64_t)(1000 * unif());
    int32_t keep[40];
    const int n = oracle_coverage_set(counts, 40, 0.9, 8, keep);
    if (n < 8 || n > 40) ++g_fail;

    const int rows = 6, K = 256;
    float* wq = fvec((size_t)rows * K, -1, 1);
    memset(wq, 0, K * sizeof(float));  /* an all-zero row */
    int8_t* q = malloc((size_t)rows * K);
    float* s = malloc((size_t)rows * (K / 32) * sizeof(float));
    if (oracle_quantize_int8_rows(wq, rows, K, q, s) != 0) ++g_fail;
    if (oracle_quantize_int4_blocks(wq, rows, K, 32, q, s) != 0) ++g_fail;
    if (oracle_quantize_int4_blocks(wq, rows, K, 128, q, s) != 0) ++g_fail;
    free(wq); free(q); free(s);

    printf("oracle under sanitizers: %d failures\n", g_fail);
    return g_fail == 0 ? 0 : 1;
}
