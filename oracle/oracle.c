/*
 * CPU oracle for the routed mixture-of-experts layer — TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library.  The product path (the HIP library and its
 * Python binding) never calls it, and it shares no code, header, table or
 * helper with that path.
 *
 * What it computes is the plain per-token definition of the layer, in double
 * precision, with every sum taken sequentially in index order.  Sources (the
 * pages this layer is described on):
 *   [K]  Kimi-Linear-48B-A3B-Instruct LiteRT-LM DETAILS.md, section
 *        "Conversion notes", bullets "Mixture of experts (26 layers)" and
 *        "Quantization of the int8 file".
 *   [Q]  litert-community/Qwen3-30B-A3B model card, "Available Artifacts"
 *        (int4 block-32 experts, fp32 scales, fp32 router) and
 *        "Conversion Notes" (the moe op computes only the 8 routed experts;
 *        softmax, top 8 and renormalisation as ordinary ops; int4 block
 *        scales below 2^-14 raised to 2^-14), "Accuracy" (activation='silu').
 *   [C]  infosave/Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made",
 *        step 3 (the noaux selection bias; restriction equals the mask).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): the selection key of the sigmoid router is sigmoid(l) + b and the
 * weights use sigmoid(l) without the bias; renormalise, then multiply by the
 * scale; no epsilon in the renormalisation; flat top-k; ties go to the lower
 * expert index; the softmax router selects on the probabilities; the FFN is
 * down(act(gate x) * (up x)) with act = silu unless gelu_tanh is asked for; the
 * int4 block runs along the input axis; the clamp is max(s, 2^-14) for either
 * int4 block width; the shared expert is added unweighted.
 *
 * The top-k decision is taken on keys rounded to fp32, the precision the
 * pages give the router (fp32 router in [Q]; fp32 activations in [K]), so
 * that this oracle and the GPU kernels decide on the same precision.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp (no BLAS).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* elementwise functions                                               */
/* ------------------------------------------------------------------ */

/* logistic function 1 / (1 + e^-z): the router's scores in [K] are sigmoids */
double oracle_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* SiLU(z) = z * sigmoid(z): the routed experts' activation in [K] ("Conversion
 * notes", mixture-of-experts bullet) and in [Q] ("Accuracy" names silu as the
 * hidden activation) */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* GELU in its tanh form, z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))): the
 * other activation the moe op's attribute names (LiteRT-LM details, "Runtime":
 * 'gelu_tanh', legacy spelling 'gelu'). */
double oracle_gelu_tanh(double z) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* ------------------------------------------------------------------ */
/* router                                                              */
/* ------------------------------------------------------------------ */

/*
 * Select the k largest keys (fp32) of n, descending, ties to the lower index.
 * Plain repeated arg-max over the not-yet-chosen entries.
 */
static void select_topk(const float* key, int n, int k, int32_t* out, unsigned char* taken) {
    memset(taken, 0, (size_t)n);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < n; ++e) {
            if (taken[e]) continue;
            if (best < 0 || key[e] > key[best]) best = e;   /* strict: first index wins ties */
        }
        taken[best] = 1;
        out[j] = best;
    }
}

/*
 * One token of the router.
 *  logits:  l_e = sum_i Wr[e][i] * x[i]               ([K]; [Q] router in plain ops)
 *  sigmoid: s_e = sigmoid(l_e), key_e = s_e + b_e; top k by key;
 *           w_j = scale * s_{e_j} / sum_j' s_{e_j'}   ([K]: top 8 on the scores plus the
 *           correction bias, weights renormalised and scaled by 2.446; [C]: the bias is a
 *           selection bias)
 *  softmax: p = softmax(l); top k by p; w_j = scale * p_{e_j} / sum_j' p_{e_j'}
 *           ([Q] "Conversion Notes": softmax, top-8 selection and renormalisation
 *           run as ordinary ops beside the moe op)
 *  gap = key_(k) - key_(k+1) of the sorted fp32 keys (+inf when k == E).
 */
static void route_token(int router, const float* x, const float* wr, const float* bias,
                        int d, int E, int k, double scale, int32_t* idx, double* w,
                        double* gap, double* logits_out, double* l, double* s, float* key,
                        unsigned char* taken) {
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        const float* row = wr + (size_t)e * d;
        for (int i = 0; i < d; ++i) acc += (double)row[i] * (double)x[i];
        l[e] = acc;
        if (logits_out) logits_out[e] = acc;
    }
    if (router == ORACLE_ROUTER_SIGMOID_BIAS) {
        for (int e = 0; e < E; ++e) {
            s[e] = oracle_sigmoid(l[e]);
            double kap = s[e] + (bias ? (double)bias[e] : 0.0);
            key[e] = (float)kap;
        }
    } else {
        double m = l[0];
        for (int e = 1; e < E; ++e) if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) { s[e] = exp(l[e] - m); z += s[e]; }
        for (int e = 0; e < E; ++e) { s[e] = s[e] / z; key[e] = (float)s[e]; }
    }
    select_topk(key, E, k, idx, taken);
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += s[idx[j]];
    for (int j = 0; j < k; ++j) w[j] = scale * (s[idx[j]] / denom);
    if (gap) {
        if (k >= E) {
            *gap = INFINITY;
        } else {
            int nxt[1];
            /* the (k+1)-th key: best among the not-taken entries */
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || key[e] > key[best]) best = e;
            }
            nxt[0] = best;
            *gap = (double)key[idx[k - 1]] - (double)key[nxt[0]];
        }
    }
}

int oracle_route(int router, const float* x, const float* wr, const float* bias, int64_t T,
                 int d, int E, int k, float scale, int32_t* idx, double* w, double* gap,
                 double* logits) {
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E) return -1;
    if (router != ORACLE_ROUTER_SIGMOID_BIAS && router != ORACLE_ROUTER_SOFTMAX) return -1;
    int err = 0;
    #pragma omp parallel
    {
        double* l = (double*)malloc(sizeof(double) * (size_t)E);
        double* s = (double*)malloc(sizeof(double) * (size_t)E);
        float* key = (float*)malloc(sizeof(float) * (size_t)E);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        if (!l || !s || !key || !taken) {
            #pragma omp atomic write
            err = -2;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t)
                route_token(router, x + (size_t)t * d, wr, bias, d, E, k, (double)scale,
                            idx + (size_t)t * k, w + (size_t)t * k, gap ? gap + t : NULL,
                            logits ? logits + (size_t)t * E : NULL, l, s, key, taken);
        }
        free(l); free(s); free(key); free(taken);
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* permutation                                                         */
/* ------------------------------------------------------------------ */

/*
 * Group the T*k (token, slot) pairs by expert ([Q]: only the routed experts
 * are computed for each token, so each expert sees exactly the tokens that
 * chose it).  Plain counting definition: walk experts in order, and within
 * an expert the pairs in (t, j) order.
 *   offsets[e]        = first row of expert e (offsets[E] = T*k)
 *   row_token[r]      = token of row r
 *   token_row[t*k+j]  = row holding pair (t, j)
 */
int oracle_permute(const int32_t* idx, int64_t T, int k, int E, int32_t* offsets,
                   int32_t* row_token, int32_t* token_row) {
    if (T < 0 || k <= 0 || E <= 0) return -1;
    int64_t n = T * (int64_t)k;
    for (int64_t i = 0; i < n; ++i)
        if (idx[i] < 0 || idx[i] >= E) return -1;
    int64_t r = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)r;
        for (int64_t t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (idx[t * k + j] == e) {
                    row_token[r] = (int32_t)t;
                    token_row[t * k + j] = (int32_t)r;
                    ++r;
                }
    }
    offsets[E] = (int32_t)r;
    return 0;
}

/* ------------------------------------------------------------------ */
/* expert FFN                                                          */
/* ------------------------------------------------------------------ */

/*
 * Dequantised weight of row n, input column i of matrix `m` (0 = gate/up
 * [2I][d], 1 = down [d][I]) of expert e:
 *   fp32:      stored value
 *   int8_row:  q * s[e][n]                    ([K] int8 per channel: one scale per
 *                                              output row and expert, symmetric)
 *   int4_b32:  q * max(s[e][n][i/32], 2^-14)  ([Q] int4 blockwise, block 32, fp32
 *                                              scales; scales below 2^-14 raised)
 *   int4_b128: q * max(s[e][n][i/128], 2^-14) (the same with blocks of 128, the
 *                                              block width the Kimi model card
 *                                              measures against 32; the clamp
 *                                              read as applying to any block)
 * int4 codes are read unpacked, one int8 per element.
 */
static inline double weight_at(const oracle_experts* W, int m, int e, int64_t n, int64_t i) {
    int64_t rows = m == 0 ? 2LL * W->inter : (int64_t)W->d;
    int64_t cols = m == 0 ? (int64_t)W->d : (int64_t)W->inter;
    const void* q = m == 0 ? W->gu : W->dn;
    const float* s = m == 0 ? W->gu_s : W->dn_s;
    int64_t at = ((int64_t)e * rows + n) * cols + i;
    if (W->fmt == ORACLE_W_FP32) return (double)((const float*)q)[at];
    double code = (double)((const int8_t*)q)[at];
    if (W->fmt == ORACLE_W_INT8_ROW) return code * (double)s[(int64_t)e * rows + n];
    /* int4, blocks of B along the input axis */
    const int64_t B = W->fmt == ORACLE_W_INT4_B128 ? 128 : 32;
    int64_t nblk = cols / B;
    double sc = (double)s[((int64_t)e * rows + n) * nblk + i / B];
    const double floor_scale = 1.0 / 16384.0; /* 2^-14 */
    if (!(sc >= floor_scale)) sc = floor_scale;
    return code * sc;
}

/*
 * out[0..d) = FFN_e(x):  g_n = sum_i Wg[n][i] x_i,  u_n = sum_i Wu[n][i] x_i,
 *                        h_n = act(g_n) * u_n,       out_m = sum_n Wd[m][n] h_n
 * with act = silu (the default) or gelu_tanh.  Rows 0..I-1 of the gate/up
 * matrix are the gate, rows I..2I-1 the up.
 */
void oracle_ffn(const oracle_experts* W, int e, const float* x, double* out, double* h) {
    int64_t I = W->inter, d = W->d;
    for (int64_t n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        for (int64_t i = 0; i < d; ++i) g += weight_at(W, 0, e, n, i) * (double)x[i];
        for (int64_t i = 0; i < d; ++i) u += weight_at(W, 0, e, I + n, i) * (double)x[i];
        h[n] = (W->act == ORACLE_ACT_GELU_TANH ? oracle_gelu_tanh(g) : oracle_silu(g)) * u;
    }
    for (int64_t m = 0; m < d; ++m) {
        double acc = 0.0;
        for (int64_t n = 0; n < I; ++n) acc += weight_at(W, 1, e, m, n) * h[n];
        out[m] = acc;
    }
}

/* rows[r] = FFN_{expert of r}(x[row_token[r]]) for every row of every expert. */
int oracle_expert_rows(const oracle_experts* W, const float* x, const int32_t* row_token,
                       const int32_t* offsets, double* rows) {
    int64_t d = W->d;
    int64_t R = offsets[W->E];
    int err = 0;
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)W->inter);
        if (!h) {
            #pragma omp atomic write
            err = -2;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < R; ++r) {
                int e = 0;
                while (!(offsets[e] <= r && r < offsets[e + 1])) ++e;
                int64_t t = row_token ? row_token[r] : r;
                oracle_ffn(W, e, x + t * d, rows + r * d, h);
            }
        }
        free(h);
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* combine                                                             */
/* ------------------------------------------------------------------ */

/*
 * y[t] = sum_{j<k} w[t][j] * rows[token_row[t*k+j]]  (slot order)
 *        + shared[t] (weight 1, [K]: the shared expert in plain ops beside the moe op)
 *        + residual[t] (the residual add sits outside the moe op, [Q] Conversion Notes)
 */
void oracle_combine(const float* rows, const int32_t* token_row, const float* w,
                    const float* shared, const float* residual, int64_t T, int k, int d,
                    double* y) {
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += (double)w[t * k + j] * (double)rows[(int64_t)token_row[t * k + j] * d + i];
            if (shared) acc += (double)shared[t * d + i];
            if (residual) acc += (double)residual[t * d + i];
            y[t * d + i] = acc;
        }
}

/* ------------------------------------------------------------------ */
/* whole layer                                                         */
/* ------------------------------------------------------------------ */

/*
 * y[t] = sum_j w_j * FFN_{e_j}(x[t]) + FFN_shared(x[t]) for each token, in
 * slot order, with (e_j, w_j) from the router above.  Tokens are
 * independent (no capacity limit or dropping is described), so the loop over
 * tokens is a plain parallel loop.  idx, w, gap may be NULL.
 */
int oracle_layer(const oracle_layer_args* L, const float* x, int64_t T, int32_t* idx,
                 double* w, double* gap, double* y) {
    int E = L->experts.E, d = L->experts.d, k = L->k;
    if (T < 0 || k <= 0 || k > E) return -1;
    if (L->has_shared && L->shared.d != d) return -1;
    int err = 0;
    #pragma omp parallel
    {
        double* l = (double*)malloc(sizeof(double) * (size_t)E);
        double* s = (double*)malloc(sizeof(double) * (size_t)E);
        float* key = (float*)malloc(sizeof(float) * (size_t)E);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        int32_t* ti = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
        double* tw = (double*)malloc(sizeof(double) * (size_t)k);
        int64_t hmax = L->experts.inter;
        if (L->has_shared && L->shared.inter > hmax) hmax = L->shared.inter;
        double* h = (double*)malloc(sizeof(double) * (size_t)hmax);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        if (!l || !s || !key || !taken || !ti || !tw || !h || !o) {
            #pragma omp atomic write
            err = -2;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                const float* xt = x + t * d;
                double g = 0.0;
                route_token(L->router, xt, L->wr, L->bias, d, E, k, (double)L->scale, ti, tw,
                            &g, NULL, l, s, key, taken);
                double* yt = y + t * d;
                for (int i = 0; i < d; ++i) yt[i] = 0.0;
                for (int j = 0; j < k; ++j) {
                    oracle_ffn(&L->experts, ti[j], xt, o, h);
                    for (int i = 0; i < d; ++i) yt[i] += tw[j] * o[i];
                }
                if (L->has_shared) {
                    oracle_ffn(&L->shared, 0, xt, o, h);
                    for (int i = 0; i < d; ++i) yt[i] += o[i];
                }
                if (idx) for (int j = 0; j < k; ++j) idx[t * k + j] = ti[j];
                if (w) for (int j = 0; j < k; ++j) w[t * k + j] = tw[j];
                if (gap) gap[t] = g;
            }
        }
        free(l); free(s); free(key); free(taken); free(ti); free(tw); free(h); free(o);
    }
    return err;
}

/* Expert restriction (Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made",
 * steps 2 and 3): per layer, keep the smallest set of experts whose recorded
 * selection counts reach the fraction `cover` of all selections.  Taking
 * experts by descending count (equal counts: lower id first) until the running
 * sum reaches cover * total gives a smallest such set.  The set is padded in
 * the same order to at least k experts (min(k, E)), so that every token can
 * still select k, and is written to keep[] in ascending id order (the dense
 * renumbering keeps the original order).  Returns its size, or -1 for bad
 * arguments (E < 1, k < 1, cover outside [0, 1]). */
int oracle_coverage_set(const uint64_t* counts, int E, double cover, int k, int32_t* keep) {
    if (E < 1 || k < 1 || !(cover >= 0.0 && cover <= 1.0)) return -1;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    if (!taken) return -2;
    uint64_t total = 0;
    for (int e = 0; e < E; ++e) total += counts[e];
    const double need = cover * (double)total;
    const int kmin = k < E ? k : E;
    uint64_t sum = 0;
    int n = 0;
    while (n < E && ((double)sum < need || n < kmin)) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || counts[e] > counts[best])) best = e;
        taken[best] = 1;
        sum += counts[best];
        ++n;
    }
    int m = 0;
    for (int e = 0; e < E; ++e)
        if (taken[e]) keep[m++] = e;
    free(taken);
    return n;
}

/* Weight quantizers: the step that produces the expert formats from float
 * weights.
 *
 * int8 per output row (Kimi-Linear-48B-A3B-Instruct LiteRT-LM details,
 * "Conversion notes", quantization of the int8 file: one scale per output row
 * and expert, symmetric min-max): s = max_k |w[k]| / 127, q[k] = round(w[k] / s),
 * so the largest magnitude maps to +-127.  An all-zero row gets s = 0 and
 * codes 0.
 *
 * int4 per block of B = 32 inputs (Qwen3-30B-A3B model card, file table:
 * int4 blockwise, block 32, fp32 scales; "Conversion notes": block scales below
 * 2^-14 are raised to 2^-14), or B = 128: s = max(max_b |w| / 7, 2^-14) over
 * the block,
 * q = round(w / s) in [-8, 7] (symmetric: at most 7 in magnitude).  Raising
 * the scale here, before dividing, makes the stored scale the one the layer
 * dequantises with.
 *
 * The pages fix no precision for the scale and the quotient.  A code is an
 * integer decided by floating point, so both are taken in fp32, each
 * correctly rounded (computed here in fp64 and rounded once to fp32, which
 * equals the correctly rounded fp32 quotient of two fp32 values), and the
 * quotient is rounded to the nearest integer with halves away from zero (C's
 * round).  Inputs must be finite. */
static inline float div_f32(float a, float b) { return (float)((double)a / (double)b); }

int oracle_quantize_int8_rows(const float* w, int64_t rows, int K, int8_t* q, float* s) {
    if (rows < 0 || K < 1) return -1;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* wr = w + r * K;
        float m = 0.0f;
        for (int k = 0; k < K; ++k) m = fabsf(wr[k]) > m ? fabsf(wr[k]) : m;
        const float sc = div_f32(m, 127.0f);
        s[r] = sc;
        for (int k = 0; k < K; ++k) {
            double c = sc > 0.0f ? round((double)div_f32(wr[k], sc)) : 0.0;
            c = c > 127.0 ? 127.0 : (c < -127.0 ? -127.0 : c);
            q[r * K + k] = (int8_t)c;
        }
    }
    return 0;
}

int oracle_quantize_int4_blocks(const float* w, int64_t rows, int K, int B, int8_t* q,
                                float* s) {
    if (rows < 0 || (B != 32 && B != 128) || K < B || K % B != 0) return -1;
    const int nb = K / B;
    const float floor_s = 1.0f / 16384.0f;  /* 2^-14 */
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float* wb = w + r * K + (int64_t)B * b;
            float m = 0.0f;
            for (int i = 0; i < B; ++i) m = fabsf(wb[i]) > m ? fabsf(wb[i]) : m;
            float sc = div_f32(m, 7.0f);
            if (sc < floor_s) sc = floor_s;
            s[r * nb + b] = sc;
            for (int i = 0; i < B; ++i) {
                double c = round((double)div_f32(wb[i], sc));
                c = c > 7.0 ? 7.0 : (c < -8.0 ? -8.0 : c);
                q[r * K + (int64_t)B * b + i] = (int8_t)c;
            }
        }
    }
    return 0;
}
