// Argument checks of the C ABI (include/moe.h), one per call.  Plain host
// C++, no HIP: each entry point runs its check before it touches the device or
// enqueues anything, and the CPU tests run the same checks without a GPU.
// Each returns MOE_OK or the status of the first problem found and writes a
// message naming the argument into err (kErrBytes bytes).  A check returns
// MOE_OK without looking at the data pointers when the call has nothing to
// do (T == 0 and the like); the caller returns at once in that case.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr size_t kErrBytes = 512;

moe_status errorf(char* err, moe_status st, const char* fmt, ...)
    __attribute__((format(printf, 3, 4)));

moe_status check_workspace_size(char* err, int T, int k, int E, int d, int inter, int fmt,
                                const size_t* bytes);
moe_status check_route(char* err, int router, const float* x, const float* w_router,
                       const float* bias, int T, int d, int E, int k, float scale,
                       const int32_t* topk_idx, const float* topk_w, const void* ws,
                       size_t ws_bytes);
moe_status check_expert_counts(char* err, const int32_t* topk_idx, int T, int k, int E,
                               const unsigned long long* counts);
moe_status check_quantize(char* err, int fmt, int in_type, const void* w, long long rows, int K,
                          const void* codes, const float* scales);
moe_status check_permute(char* err, const int32_t* topk_idx, int T, int k, int E,
                         const int32_t* offsets, const int32_t* row_token,
                         const int32_t* token_row);
moe_status check_weights(char* err, const char* fn, const char* which, const moe_weights* w);
moe_status check_expert_ffn(char* err, const moe_weights* w, int act, const float* x, int T,
                            const int32_t* row_token, const int32_t* offsets, int R_max,
                            const float* rows_out, const void* ws, size_t ws_bytes);
moe_status check_layer(char* err, const char* fn, const moe_layer* L);
moe_status check_layer_workspace_size(char* err, const moe_layer* L, int T, const size_t* bytes);
// cu_count: the device's compute units (the small-batch launch plan depends on it)
// fn: the entry point's name for the messages (moe_forward, moe_forward_noalloc)
moe_status check_forward(char* err, const char* fn, const moe_layer* L, int act, const float* x,
                         int T, const float* residual, const float* y, const int32_t* topk_idx,
                         const float* topk_w, const void* ws, size_t ws_bytes, int cu_count);
moe_status check_forward_chained(char* err, const moe_layer* L, int act, const float* x,
                                 const moe_pending* in, const float* x_out, int T,
                                 const moe_pending* out, const int32_t* topk_idx,
                                 const float* topk_w, const void* ws, size_t ws_bytes,
                                 int cu_count);
moe_status check_tile_weights(char* err, const moe_weights* src, const void* dst_gate_up,
                              const void* dst_down);
moe_status check_combine(char* err, const float* rows, const int32_t* token_row,
                         const float* topk_w, const float* shared, const float* residual, int T,
                         int k, int d, const float* y);
moe_status check_coverage_set(char* err, const unsigned long long* counts, int E, double cover,
                              int k, const int32_t* keep, const int32_t* n_keep);
moe_status check_probe_read(char* err, const void* buf, size_t bytes, int blocks,
                            const void* sink);
moe_status check_probe_mfma(char* err, int shape, int iters, int blocks, const void* sink);
constexpr int kProbeMaxBlocks = 1 << 20;

// Whether moe_forward at T tokens runs the small-batch path (the router
// encodes x and the FFN kernels group the pairs themselves).
bool forward_small(const moe_layer* L, int T);

}  // namespace moe
