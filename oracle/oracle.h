/*
 * CPU oracle for the routed mixture-of-experts layer — TEST INFRASTRUCTURE.
 * Declarations for oracle.c; used only by oracle/__init__.py (ctypes).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_ROUTER_SIGMOID_BIAS = 0, ORACLE_ROUTER_SOFTMAX = 1 };
enum { ORACLE_W_FP32 = 0, ORACLE_W_INT8_ROW = 1, ORACLE_W_INT4_B32 = 2, ORACLE_W_INT4_B128 = 3 };
enum { ORACLE_ACT_SILU = 0, ORACLE_ACT_GELU_TANH = 1 };

/* Experts in one format.  int4 codes are unpacked (one int8 per element). */
typedef struct {
    int fmt;
    int E, d, inter;
    const void* gu;      /* [E][2I][d]  fp32 or int8 codes                     */
    const float* gu_s;   /* int8: [E][2I]; int4: [E][2I][d/B] (B = 32 or 128)  */
    const void* dn;      /* [E][d][I]                                          */
    const float* dn_s;   /* int8: [E][d];  int4: [E][d][I/B]                   */
    int act;             /* ORACLE_ACT_*: the activation of the gate            */
} oracle_experts;

typedef struct {
    int router;
    int k;
    float scale;
    const float* wr;     /* [E][d] */
    const float* bias;   /* [E] or NULL */
    oracle_experts experts;
    int has_shared;
    oracle_experts shared; /* E == 1 */
} oracle_layer_args;

double oracle_sigmoid(double z);
double oracle_silu(double z);
double oracle_gelu_tanh(double z);
int oracle_route(int router, const float* x, const float* wr, const float* bias, int64_t T,
                 int d, int E, int k, float scale, int32_t* idx, double* w, double* gap,
                 double* logits);
int oracle_permute(const int32_t* idx, int64_t T, int k, int E, int32_t* offsets,
                   int32_t* row_token, int32_t* token_row);
void oracle_ffn(const oracle_experts* W, int e, const float* x, double* out, double* h);
int oracle_expert_rows(const oracle_experts* W, const float* x, const int32_t* row_token,
                       const int32_t* offsets, double* rows);
void oracle_combine(const float* rows, const int32_t* token_row, const float* w,
                    const float* shared, const float* residual, int64_t T, int k, int d,
                    double* y);
int oracle_layer(const oracle_layer_args* L, const float* x, int64_t T, int32_t* idx,
                 double* w, double* gap, double* y);
int oracle_coverage_set(const uint64_t* counts, int E, double cover, int k, int32_t* keep);
int oracle_quantize_int8_rows(const float* w, int64_t rows, int K, int8_t* q, float* s);
int oracle_quantize_int4_blocks(const float* w, int64_t rows, int K, int B, int8_t* q, float* s);

#ifdef __cplusplus
}
#endif
#endif
