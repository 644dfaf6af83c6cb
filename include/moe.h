/*
 * moe.h — C ABI of the MI355X (gfx950) routed mixture-of-experts layer.
 *
 * The layer, per token x (fp32, length d):
 *   1. router logits l = Wr x (Wr: E x d, fp32);
 *   2. selection of k experts and their weights (moe_route);
 *   3. grouping of the (token, slot) pairs by expert (moe_permute);
 *   4. each selected expert's SwiGLU FFN, weights dequantised in-kernel
 *      (moe_expert_ffn; the shared expert is one more call with one expert);
 *   5. y = sum_j w_j * FFN_{e_j}(x) + shared(x) [+ residual] (moe_combine).
 * Sources: the Kimi-Linear-48B-A3B-Instruct LiteRT-LM DETAILS.md ("Conversion
 * notes": the mixture-of-experts and int8-quantization bullets; "Runtime": an
 * unsupported activation is rejected at setup with a message) and the
 * litert-community Qwen3-30B-A3B model card ("Available Artifacts": int4
 * block-32 experts with fp32 scales, fp32 router; "Conversion Notes": the
 * moe op computes only the routed experts, softmax/top-8/renormalisation,
 * scales below 2^-14 raised to 2^-14, residual add outside the op).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns all
 *    memory; the library allocates nothing on the call path.  Every device
 *    pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *    and return without synchronising the host; data-dependent sizes (how
 *    many rows each expert received) stay on the device.
 *  - Errors are return codes; nothing aborts or throws across the ABI.  All
 *    argument checks are host code and run before anything is enqueued
 *    (including moe_forward's check that its small-batch launch plan fits the
 *    workspace's split-K join area); on failure nothing is launched and
 *    moe_last_error() names the argument.
 *  - T == 0 is a valid no-op.  A moe_ctx must not be used by two host
 *    threads at once.  Work enqueued on one stream runs in order; calls that
 *    share a workspace must not overlap on different streams.
 *  - Results are deterministic: the same inputs give the same bits on every
 *    run, and a token's router logits do not depend on T.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;

typedef enum {
    MOE_OK = 0,
    MOE_E_INVALID = 1,      /* a bad argument (null, negative, misaligned, k > E ...)      */
    MOE_E_UNSUPPORTED = 2,  /* valid but not implemented (other activation, odd sizes ...) */
    MOE_E_DEVICE = 3,       /* a HIP runtime error; the message carries HIP's text          */
    MOE_E_WORKSPACE = 4     /* workspace pointer NULL or smaller than moe_workspace_size   */
} moe_status;

typedef enum {
    /* sigmoid scores s = 1/(1+exp(-l)); top k on s + bias; w = scale * s / sum(s)
       (DETAILS.md, Conversion notes, mixture-of-experts bullet; scale 2.446) */
    MOE_ROUTER_SIGMOID_BIAS = 0,
    /* p = softmax(l) over all E; top k on p; w = scale * p / sum(p) (Qwen3 card,
       Conversion Notes; scale 1) */
    MOE_ROUTER_SOFTMAX = 1
} moe_router;

typedef enum {
    MOE_W_FP32 = 0,      /* plain fp32 weights, no scales                              */
    MOE_W_INT8_ROW = 1,  /* int8 codes, one fp32 scale per output row and expert:
                            w = q * s[row] (DETAILS.md, quantization of the int8 file) */
    MOE_W_INT4_B32 = 2,  /* int4 codes in blocks of 32 along the input axis with fp32
                            scales raised to 2^-14: w = q * max(s[row][i/32], 2^-14)
                            (Qwen3 card, Available Artifacts and Conversion Notes).
                            Two codes per byte, two's complement: input element 2i in
                            the low nibble of byte i, element 2i+1 in the high nibble */
    MOE_W_INT4_B128 = 3  /* the same codes with one scale per block of 128 inputs:
                            w = q * max(s[row][i/128], 2^-14) (the 128-wide blocks the
                            Kimi-Linear LiteRT-LM model card measures beside 32-wide
                            ones; the 2^-14 floor read as applying to any block) */
} moe_wfmt;

typedef enum {
    MOE_ACT_SILU = 0,     /* h = silu(gate x) * (up x), silu(z) = z / (1 + exp(-z)) */
    MOE_ACT_GELU_TANH = 1 /* h = gelu(gate x) * (up x) with the tanh form
                             gelu(z) = z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
                             (DETAILS.md, Runtime: the moe op's activation attribute
                             is 'silu' or 'gelu_tanh', legacy spelling 'gelu') */
} moe_act;

/* Byte order of the int8/int4 codes in HBM (scales are always row-major).
 * MOE_LAYOUT_ROWS:  [E][N][K] codes, input axis contiguous (int4: K/2 bytes per row).
 * MOE_LAYOUT_TILED: the same bytes regrouped as matrix-core operands, so that a
 *   wavefront streams whole 1 KB blocks: per expert, for each group of 16 rows
 *   (n/16) and each 64-wide input step (int8; int4: each 128-wide span) one
 *   1 KB block in lane order, lane = n%16 + 16*g.  int8: g = (k%64)/16, the lane
 *   holds k%16 = 0..15.  int4: g = (k%32)/8, the lane holds 4 bytes per block of
 *   32 (its 8 codes, two per byte, low nibble first) for the span's 4 blocks.
 *   moe_tile_weights converts; it is the faster layout for every shape. */
typedef enum {
    MOE_LAYOUT_ROWS = 0,
    MOE_LAYOUT_TILED = 1
} moe_layout;

/* A set of SwiGLU experts.  [host] struct holding device pointers.
 *   fmt        one of moe_wfmt
 *   layout     one of moe_layout (MOE_LAYOUT_ROWS for fp32)
 *   n_experts  E >= 1
 *   d          model width; a multiple of 64 (int4, either block: of 128), at
 *              most 16384
 *   inter      expert intermediate width I; a multiple of 64 (int4: of 128), at
 *              most 16384
 *   w_gate_up  [E][2I][d]: rows 0..I-1 are the gate projection, rows I..2I-1 the
 *              up projection, input axis contiguous.  int8: int8_t; int4: uint8_t
 *              with d/2 bytes per row; fp32: float
 *   s_gate_up  int8: [E][2I]; int4: [E][2I][d/32] (block 128: [E][2I][d/128]);
 *              fp32: NULL
 *   w_down     [E][d][I] (int4: [E][d][I/2] bytes)
 *   s_down     int8: [E][d]; int4: [E][d][I/32] (block 128: [E][d][I/128]); fp32:
 *              NULL                                                                  */
typedef struct {
    int fmt;
    int layout;
    int n_experts;
    int d;
    int inter;
    const void* w_gate_up;
    const float* s_gate_up;
    const void* w_down;
    const float* s_down;
} moe_weights;

/* Element type of float weights handed to moe_quantize. */
typedef enum {
    MOE_IN_F32 = 0,   /* fp32                                        */
    MOE_IN_BF16 = 1   /* bf16 (the upper 16 bits of an fp32), widened exactly */
} moe_in_type;

/* Quantize float weights on the device into one of the expert formats, row
 * layout (MOE_LAYOUT_ROWS; moe_tile_weights converts afterwards).  w is a
 * [rows][K] matrix with the input axis contiguous: for an expert set, the
 * gate/up codes are rows = E*2I, K = d and the down codes rows = E*d, K = I.
 *   MOE_W_INT8_ROW (Kimi-Linear-48B-A3B-Instruct LiteRT-LM details,
 *     "Conversion notes", quantization of the int8 file: symmetric min-max,
 *     one scale per output row):  scales[r] = max_k |w[r][k]| / 127,
 *     codes[r][k] = round(w[r][k] / scales[r]) as int8 in [-127, 127]; an
 *     all-zero row gets scale 0 and codes 0.  K a multiple of 8.
 *   MOE_W_INT4_B32 (Qwen3-30B-A3B model card: int4 blockwise, block 32, fp32
 *     scales; block scales below 2^-14 raised to 2^-14):
 *     scales[r][b] = max(max_{k in block b} |w[r][k]| / 7, 2^-14),
 *     codes in [-7, 7], two per byte ([rows][K/2] bytes, low nibble = even k).
 *     K a multiple of 32.
 *   MOE_W_INT4_B128: the same per block of 128 (scales [rows][K/128]); K a
 *     multiple of 128.
 * Both divisions are correctly rounded fp32; the quotient is rounded to the
 * nearest integer, halves away from zero.  Inputs must be finite.
 *   in_type  one of moe_in_type
 *   codes    int8 [rows][K] or uint8 [rows][K/2]; scales fp32 [rows] or
 *            [rows][K/32]; caller-owned, 16-byte aligned, not overlapping w.
 * K above 2^24, rows above 2^32 or rows*K above 2^40 returns MOE_E_UNSUPPORTED.  Enqueued on
 * `stream`; one read of w and one write of the codes and scales. */
moe_status moe_quantize(moe_ctx* ctx, int fmt, int in_type, const void* w, long long rows,
                        int K, void* codes, float* scales, void* stream);

/* Copy row-major int8/int4 codes into MOE_LAYOUT_TILED order (a byte
 * permutation; scales are not touched).  src: weights with layout
 * MOE_LAYOUT_ROWS; dst_gate_up / dst_down: device buffers of the same byte
 * sizes as src's codes, not overlapping them.  Enqueued on `stream`.  For a
 * one-time conversion at load; the result is used with the same scales and
 * layout = MOE_LAYOUT_TILED. */
moe_status moe_tile_weights(moe_ctx* ctx, const moe_weights* src, void* dst_gate_up,
                            void* dst_down, void* stream);

/* Context on HIP device `device`; reads its properties once.  [host] *out. */
moe_status moe_create(int device, moe_ctx** out);
void moe_destroy(moe_ctx* ctx);

/* Message for the last failed call on this context ("" if none).  The pointer
   stays valid until the next call on the context.  With ctx == NULL, the
   message of the last moe_create failure in this process. */
const char* moe_last_error(const moe_ctx* ctx);
const char* moe_status_string(moe_status status);

/* Bytes of device workspace that moe_route and moe_expert_ffn need
   for a layer of T tokens, top k of E experts, width d, intermediate width
   `inter` and weight format `fmt` (the larger of the two calls; one buffer
   may serve all of them in turn on one stream).  [host] *bytes.
   For the shared expert (one expert over T rows) pass k = 1, E = 1.
   For int8/int4 weights this includes about 16 MB where small decode
   launches that split K across workgroups meet (partial sums and arrival
   counts); the workspace needs no initialisation, each call clears the
   counts it uses before its FFN kernels run. */
moe_status moe_workspace_size(const moe_ctx* ctx, int T, int k, int E, int d, int inter,
                              int fmt, size_t* bytes);

/* Router (DETAILS.md, mixture-of-experts bullet; Qwen3 card, Conversion Notes).
 *   x         [T][d] fp32 activations
 *   w_router  [E][d] fp32
 *   bias      [E] fp32 selection bias (sigmoid router; NULL = zero); must be NULL
 *             for the softmax router
 *   k         1 <= k <= min(E, 16); E <= 1024; d a multiple of 64, at most 16384
 *   scale     multiplies the renormalised weights (2.446 for the Kimi-style
 *             sigmoid router, 1 for softmax); finite
 *   topk_idx  [T][k] int32 out: expert ids by descending selection key, ties to
 *             the lower id
 *   topk_w    [T][k] fp32 out: weights, same order
 * The logits are fp32 sums in a fixed order per token; the selection keys are
 * fp32. */
moe_status moe_route(moe_ctx* ctx, int router, const float* x, const float* w_router,
                     const float* bias, int T, int d, int E, int k, float scale,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream);

/* Router restricted to a subset of the experts.  Restricting a model to an
 * expert subset is the same as masking the others at run time
 * (Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made", step 3): the
 * result equals moe_route on the allowed experts alone (router rows and bias
 * sliced, ids mapped back), bit for bit.
 *   mask  [E] uint8 device array: nonzero = the expert may be selected, 0 =
 *         never; NULL = all allowed (then this is moe_route).  At least k experts
 *         should be allowed: with fewer, the remaining slots hold masked experts
 *         (lowest id first, ids still in [0, E)) with weight 0, and with none
 *         allowed every weight is NaN.  Sigmoid router: masked experts drop out
 *         of the selection and their scores never enter a weight.  Softmax
 *         router: the softmax runs over the allowed experts only.
 * Other arguments, checks and errors as for moe_route. */
moe_status moe_route_masked(moe_ctx* ctx, int router, const float* x, const float* w_router,
                            const float* bias, const uint8_t* mask, int T, int d, int E,
                            int k, float scale, int32_t* topk_idx, float* topk_w, void* ws,
                            size_t ws_bytes, void* stream);

/* Routing statistics (the per-expert routing frequencies of the
 * Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made", step 2):
 *   counts[e] += #{(t, j) : topk_idx[t][j] == e}   for e < E
 *   topk_idx [T][k] int32 device; counts [E] uint64 device, accumulated (the
 *   caller zeroes it once).  Entries outside [0, E) are not counted. */
moe_status moe_expert_counts(moe_ctx* ctx, const int32_t* topk_idx, int T, int k, int E,
                             unsigned long long* counts, void* stream);

/* Expert restriction (Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made",
 * step 3): from the selection counts a calibration run recorded (moe_expert_counts),
 * the smallest set of experts that carries the share `cover` of all selections.
 * Experts are taken by descending count, equal counts by ascending id, until
 * the running sum reaches cover * total (the comparison in double precision:
 * (double) running >= cover * (double) total; none is needed when that product
 * is 0); the set is then padded in the same order to min(k, E) experts so that
 * a token can still select k.
 *   counts  [E] uint64 device (E in [1, 1024]); cover in [0, 1]; k >= 1
 *   keep    [E] int32 device out: the kept ids ascending in keep[0..n-1], -1 after
 *   n_keep  [1] int32 device out: n
 * One workgroup, asynchronous on `stream`.  Errors: MOE_E_INVALID for E, k
 * or cover out of range and NULL or misaligned pointers (16-byte alignment);
 * nothing is launched on an error. */
moe_status moe_coverage_set(moe_ctx* ctx, const unsigned long long* counts, int E, double cover,
                            int k, int32_t* keep, int32_t* n_keep, void* stream);

/* Group the T*k (token, slot) pairs by expert (Qwen3 card, Conversion Notes:
 * only the routed experts are computed for each token).  Stable: within an
 * expert, rows follow (t, j) order.
 *   topk_idx   [T][k] int32 in [0, E) (entries outside are given no row and
 *              their token_row is -1)
 *   offsets    [E+1] out: rows of expert e are offsets[e] .. offsets[e+1]-1
 *   row_token  [T*k] out: token of each row
 *   token_row  [T*k] out: row of pair (t, j) at index t*k + j                     */
moe_status moe_permute(moe_ctx* ctx, const int32_t* topk_idx, int T, int k, int E,
                       int32_t* offsets, int32_t* row_token, int32_t* token_row, void* stream);

/* Expert SwiGLU FFNs over grouped rows (DETAILS.md, mixture-of-experts bullet:
 * the routed experts with SiLU; Qwen3 card, Accuracy: activation 'silu').
 *   rows_out[r] = W_down[e] (act(W_gate[e] x[row_token[r]]) * W_up[e] x[row_token[r]])
 * for every row r of every expert e, with weights dequantised in-kernel.
 *   act        MOE_ACT_SILU or MOE_ACT_GELU_TANH; anything else returns
 *              MOE_E_UNSUPPORTED with a message
 *   x          [T][d] fp32
 *   row_token  [R] or NULL (row r reads token r)
 *   offsets    [E+1] device, as written by moe_permute; NULL only when E == 1,
 *              meaning one expert over rows 0 .. R_max-1
 *   R_max      number of rows the caller sized rows_out for (T*k for routed
 *              experts, T for the shared expert); offsets[E] must not exceed it
 *   rows_out   [R_max][d] fp32 out (rows beyond offsets[E] are not written)    */
moe_status moe_expert_ffn(moe_ctx* ctx, const moe_weights* w, int act, const float* x, int T,
                          const int32_t* row_token, const int32_t* offsets, int R_max,
                          float* rows_out, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine (DETAILS.md, mixture-of-experts bullet: routed experts and
 * the shared expert; Qwen3 card, Conversion Notes: the residual add sits after
 * the moe op).
 *   y[t] = sum_{j<k} topk_w[t][j] * rows[token_row[t*k+j]]  (slot order)
 *          + shared[t] (if not NULL) + residual[t] (if not NULL)
 *   rows [R][d], token_row [T*k] (NULL: rows already in (token, slot) order, row
 *   t*k + j), topk_w [T][k], shared/residual/y [T][d] fp32.
 *   y may alias residual.                                                          */
moe_status moe_combine(moe_ctx* ctx, const float* rows, const int32_t* token_row,
                       const float* topk_w, const float* shared, const float* residual,
                       int T, int k, int d, float* y, void* stream);

/* A whole layer for moe_forward.  [host] struct holding device pointers.
 *   router, k, scale, w_router [E][d], bias [E] or NULL: as for moe_route
 *   experts: the routed experts (E = experts.n_experts)
 *   shared:  the shared expert (shared.n_experts == 1), or shared.n_experts == 0
 *            for none; same d as the routed experts
 *   expert_mask: [E] uint8 device, or NULL; restricts the routed experts as in
 *            moe_route_masked                                                   */
typedef struct {
    int router;
    int k;
    float scale;
    const float* w_router;
    const float* bias;
    moe_weights experts;
    moe_weights shared;
    const uint8_t* expert_mask;  /* [E] device, or NULL: see moe_route_masked */
} moe_layer;

/* Workspace for moe_forward on T tokens (as moe_workspace_size, including the
   split-K area for int8/int4 layers).  [host] *bytes. */
moe_status moe_layer_workspace_size(const moe_ctx* ctx, const moe_layer* layer, int T,
                                    size_t* bytes);

/* The whole layer in one call: the same result, bit for bit in the router
 * outputs and to rounding in y, as moe_route, moe_permute, moe_expert_ffn on
 * the routed experts, moe_expert_ffn on the shared expert and moe_combine in
 * turn (DETAILS.md, mixture-of-experts bullet: routed experts weighted by the
 * router, shared expert added; the residual is added after the moe op, Qwen3
 * card, Conversion Notes).  Fewer launches: x is encoded once and, when the
 * shared expert has the routed experts' format, its tiles run inside the
 * routed experts' launches.
 *   x [T][d], residual [T][d] or NULL, y [T][d] out (may alias residual)
 *   topk_idx [T][k], topk_w [T][k]: outputs, or NULL to keep them internal
 *   act: the gate activation of the routed and the shared experts alike
 * Checks and errors as for the separate calls. */
moe_status moe_forward(moe_ctx* ctx, const moe_layer* layer, int act, const float* x, int T,
                       const float* residual, float* y, int32_t* topk_idx, float* topk_w,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It runs exactly moe_forward's kernels, with the
 * library's own scratch array (a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process ends)
 * as the workspace; it allocates nothing.  Every call on a GPU shares that
 * GPU's array and leaves its contents behind, so calls that overlap on one GPU
 * (on two streams, or from two threads) race: serialise them.  A layer whose
 * moe_layer_workspace_size at T exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 * MOE_E_UNSUPPORTED before anything is enqueued (40 MiB covers a Kimi-shaped
 * layer, d = 2304, E = 256, I = 2048 with its int8 shared expert, up to
 * T = 186, and a Qwen-shaped int4 layer, d = 2048, E = 128, I = 768, up to
 * T = 290).  Arguments, checks, results and other errors as for
 * moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (40u * 1024u * 1024u)
moe_status moe_forward_noalloc(moe_ctx* ctx, const moe_layer* layer, int act, const float* x,
                               int T, const float* residual, float* y, int32_t* topk_idx,
                               float* topk_w, void* stream);

/* Layers chained without a combine launch between them (decode-size stacks,
 * x_{l+1} = x_l + MoE_l(x_l); Qwen3-30B-A3B model card, "Conversion Notes":
 * the residual add follows the moe op).  A layer's output, y = sum over slots
 * j of w[t][j] * rows[t*k + j] (slot order) + shared[t] + residual[t], is the
 * combine of moe_combine; it can be left pending and formed by the next
 * layer's router launch, which reads x anyway: one launch fewer per layer.
 * moe_forward_chained runs the layer as moe_forward does, except that
 *   - its input is x (in == NULL), or the pending output `in` of the previous
 *     chained call (x == NULL), which the router launch sums exactly as
 *     moe_combine would and stores into x_out [T][d] (device, 16-byte
 *     aligned, overlapping none of in's arrays): x_out is the layer's input
 *     from then on, bit for bit the y an unchained layer would have written;
 *   - it does not combine: it fills *out (host struct) with its own pending
 *     output: rows and shared rows in ws, the weights in topk_w (or ws), and
 *     the residual = the layer's input (x, or x_out).  They stay valid until
 *     ws, topk_w or that input is written again; complete them with
 *     moe_combine(out->rows, NULL, out->w, out->shared, out->residual, T,
 *     out->k, out->d, y) or pass them to the next chained call, which must
 *     use another workspace.
 * Only the small-batch path chains: T <= 16, quantised routed experts and,
 * if there is a shared expert, one in the routed experts' format and layout
 * (one pair of FFN launches); in (if given) must have in->T == T and
 * in->d == the layer's d.  Anything else returns MOE_E_UNSUPPORTED or
 * MOE_E_INVALID before any launch; the other checks are moe_forward's. */
typedef struct {
    const float* rows;      /* [T*k][d] routed expert rows, (token, slot) order */
    const float* shared;    /* [T][d] shared expert rows, or NULL */
    const float* w;         /* [T][k] router weights */
    const float* residual;  /* [T][d], or NULL */
    int T, k, d;
} moe_pending;
moe_status moe_forward_chained(moe_ctx* ctx, const moe_layer* layer, int act, const float* x,
                               const moe_pending* in, float* x_out, int T, moe_pending* out,
                               int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                               void* stream);

/* Attainable-peak probes, a measurement aid for benchmarks: they compute
 * nothing of the layer.  A caller times them (events on `stream`) to state
 * the ceilings the chip reaches in practice beside its published peaks.
 * moe_probe_read: one launch of `blocks` workgroups of 256 threads (0: 8 per
 * compute unit) that reads `bytes` bytes of device memory from buf (16-byte
 * aligned; bytes a multiple of 16, at least 16) in 16-byte loads, 8 in flight
 * per lane, and discards them.
 * moe_probe_mfma: one launch of `blocks` workgroups of 256 threads (0: 8 per
 * compute unit) in which every wavefront runs `iters` rounds of 32 int8
 * MFMAs (four independent accumulator chains), shape MOE_PROBE_MFMA_16X16X64
 * (32768 operations each) or MOE_PROBE_MFMA_32X32X32 (65536); a launch
 * performs blocks * 4 * iters * 32 * (operations per MFMA) int8 operations.
 * Both may write up to 16 bytes of sink (device memory, 16-byte aligned).
 * Errors: MOE_E_INVALID for NULL or misaligned pointers, sizes out of range
 * (bytes < 16 or not a multiple of 16, iters < 1, blocks < 0 or > 2^20, an
 * unknown shape), MOE_E_DEVICE if the launch fails; nothing is launched on
 * an error. */
#define MOE_PROBE_MFMA_16X16X64 0
#define MOE_PROBE_MFMA_32X32X32 1
moe_status moe_probe_read(moe_ctx* ctx, const void* buf, size_t bytes, int blocks, void* sink,
                          void* stream);
moe_status moe_probe_mfma(moe_ctx* ctx, int shape, int iters, int blocks, void* sink,
                          void* stream);

/* Kernel timing, a measurement aid for benchmarks; off by default.
 * moe_timing(ctx, capacity > 0) creates 2*capacity HIP events (host-side
 * allocation, outside any call path) and from then on has every kernel
 * launch of the calls above record its kernel's start and stop on a pair of
 * them (hipExtLaunchKernel: the dispatch's own timestamps, so the time
 * excludes the dispatch and no event packet sits between kernels); capacity
 * = 0 switches it off and frees the events.  Not for stream capture: time
 * plain runs separately.
 * moe_timing_read synchronises on the recorded events and returns, per
 * kernel that ran, the number of launches and their summed duration, then
 * forgets them; out[] receives at most max_out entries and *n_out the number
 * of kernels seen.  Launches beyond the capacity are not timed (the read
 * still returns MOE_OK and moe_last_error() says how many were missed). */
typedef struct {
    const char* name;     /* static string, e.g. "ffn_i8_gate_up" */
    long long launches;
    double total_ms;
} moe_kernel_time;

moe_status moe_timing(moe_ctx* ctx, int capacity);
moe_status moe_timing_read(moe_ctx* ctx, moe_kernel_time* out, int max_out, int* n_out);

#ifdef __cplusplus
}
#endif
#endif
