// Host-only tests of the C ABI's argument checks (the checks every entry
// point of include/moe.h runs before it touches the device; csrc/checks.cc),
// built without HIP and, from the pytest wrapper, with the address and
// undefined-behaviour sanitizers.  Pointers are stand-in addresses: the
// checks look at their values (NULL, alignment, overlap), never at the memory
// behind them.  Each case states the call, the expected status and a word the
// message must contain.  Prints the failures and a summary line; exit status 0
// iff every case holds.
#include <stdio.h>
#include <string.h>

#include "../../sparse_moe_expert_sigmoid_amd/csrc/checks.h"
#include "../../sparse_moe_expert_sigmoid_amd/csrc/layout.h"

using namespace moe;

static int g_cases = 0, g_fail = 0;
static char g_err[kErrBytes];

static void expect(const char* what, moe_status got, moe_status want, const char* word) {
  ++g_cases;
  const bool ok = got == want && (word == nullptr || strstr(g_err, word) != nullptr);
  if (!ok) {
    ++g_fail;
    printf("FAIL %s: status %d (want %d), message \"%s\" (want \"%s\")\n", what, (int)got,
           (int)want, g_err, word ? word : "");
  }
  g_err[0] = '\0';
}
#define EXPECT(call, want, word) expect(#call, call, want, word)

// stand-in device addresses: 16-byte aligned, distinct, never dereferenced
template <class T>
static T* dev(unsigned long long n) {
  return reinterpret_cast<T*>(0x10000000ull + n * 0x100000ull);
}
template <class T>
static T* misaligned(unsigned long long n) {
  return reinterpret_cast<T*>(0x10000000ull + n * 0x100000ull + 4);
}

static moe_weights int8_experts(int E, int d, int I) {
  moe_weights w{};
  w.fmt = MOE_W_INT8_ROW;
  w.layout = MOE_LAYOUT_TILED;
  w.n_experts = E;
  w.d = d;
  w.inter = I;
  w.w_gate_up = dev<void>(1);
  w.s_gate_up = dev<float>(2);
  w.w_down = dev<void>(3);
  w.s_down = dev<float>(4);
  return w;
}

static moe_layer kimi_layer() {
  moe_layer L{};
  L.router = MOE_ROUTER_SIGMOID_BIAS;
  L.k = 8;
  L.scale = 2.446f;
  L.w_router = dev<float>(5);
  L.bias = dev<float>(6);
  L.experts = int8_experts(256, 2304, 2048);
  L.shared = int8_experts(1, 2304, 2048);
  L.shared.w_gate_up = dev<void>(7);
  L.shared.w_down = dev<void>(8);
  return L;
}

static void route_cases() {
  const float* x = dev<float>(10);
  const float* wr = dev<float>(11);
  const float* b = dev<float>(12);
  int32_t* idx = dev<int32_t>(13);
  float* w = dev<float>(14);
  void* ws = dev<void>(15);
  const size_t need = route_ws_bytes(8, 2304, 256);
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 256, 8, 2.446f, idx, w, ws, need), MOE_OK,
         nullptr);
  EXPECT(check_route(g_err, 2, x, wr, b, 8, 2304, 256, 8, 2.446f, idx, w, ws, need),
         MOE_E_INVALID, "router");
  EXPECT(check_route(g_err, 0, x, wr, b, -1, 2304, 256, 8, 2.446f, idx, w, ws, need),
         MOE_E_INVALID, "T=-1");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 256, 17, 2.446f, idx, w, ws, need),
         MOE_E_INVALID, "k=17");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 4, 8, 2.446f, idx, w, ws, need),
         MOE_E_INVALID, "k=8");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 2000, 8, 2.446f, idx, w, ws, need),
         MOE_E_INVALID, "E=2000");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2300, 256, 8, 2.446f, idx, w, ws, need),
         MOE_E_UNSUPPORTED, "multiple of 64");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 256, 8, 1.0f / 0.0f, idx, w, ws, need),
         MOE_E_INVALID, "scale");
  EXPECT(check_route(g_err, 1, x, wr, b, 8, 2304, 256, 8, 1.0f, idx, w, ws, need),
         MOE_E_INVALID, "bias");
  EXPECT(check_route(g_err, 0, nullptr, wr, b, 8, 2304, 256, 8, 2.446f, idx, w, ws, need),
         MOE_E_INVALID, "x is NULL");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 256, 8, 2.446f, nullptr, w, ws, need),
         MOE_E_INVALID, "topk_idx is NULL");
  EXPECT(check_route(g_err, 0, misaligned<float>(10), wr, b, 8, 2304, 256, 8, 2.446f, idx, w,
                     ws, need),
         MOE_E_INVALID, "aligned");
  EXPECT(check_route(g_err, 0, x, wr, misaligned<float>(12), 8, 2304, 256, 8, 2.446f, idx, w,
                     ws, need),
         MOE_E_INVALID, "aligned");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 256, 8, 2.446f, idx, w, ws, need - 1),
         MOE_E_WORKSPACE, "too small");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 256, 8, 2.446f, idx, w, nullptr, need),
         MOE_E_WORKSPACE, "NULL");
  EXPECT(check_route(g_err, 0, x, wr, b, 8, 2304, 256, 8, 2.446f, idx, w, misaligned<void>(15),
                     need),
         MOE_E_WORKSPACE, "aligned");
  // T = 0: a no-op, whatever the data pointers
  EXPECT(check_route(g_err, 0, nullptr, nullptr, nullptr, 0, 2304, 256, 8, 2.446f, nullptr,
                     nullptr, nullptr, 0),
         MOE_OK, nullptr);
}

static void permute_counts_cases() {
  const int32_t* idx = dev<int32_t>(20);
  int32_t* off = dev<int32_t>(21);
  int32_t* rt = dev<int32_t>(22);
  int32_t* tr = dev<int32_t>(23);
  EXPECT(check_permute(g_err, idx, 8, 8, 256, off, rt, tr), MOE_OK, nullptr);
  EXPECT(check_permute(g_err, idx, -3, 8, 256, off, rt, tr), MOE_E_INVALID, "T=-3");
  EXPECT(check_permute(g_err, idx, 8, 17, 256, off, rt, tr), MOE_E_INVALID, "k=17");
  EXPECT(check_permute(g_err, idx, 8, 8, 0, off, rt, tr), MOE_E_INVALID, "E=0");
  EXPECT(check_permute(g_err, idx, 8, 8, 256, nullptr, rt, tr), MOE_E_INVALID, "offsets");
  EXPECT(check_permute(g_err, idx, 8, 8, 256, off, nullptr, tr), MOE_E_INVALID, "row_token");
  EXPECT(check_permute(g_err, idx, 8, 8, 256, off, rt, misaligned<int32_t>(23)), MOE_E_INVALID,
         "aligned");
  EXPECT(check_permute(g_err, idx, 0x40000000, 8, 256, off, rt, tr), MOE_E_INVALID, "overflows");
  EXPECT(check_permute(g_err, nullptr, 0, 8, 256, off, nullptr, nullptr), MOE_OK, nullptr);
  unsigned long long* cnt = dev<unsigned long long>(24);
  EXPECT(check_expert_counts(g_err, idx, 8, 8, 256, cnt), MOE_OK, nullptr);
  EXPECT(check_expert_counts(g_err, idx, -1, 8, 256, cnt), MOE_E_INVALID, "T=-1");
  EXPECT(check_expert_counts(g_err, idx, 8, 8, 1025, cnt), MOE_E_INVALID, "E=1025");
  EXPECT(check_expert_counts(g_err, idx, 8, 8, 256, nullptr), MOE_E_INVALID, "counts");
  EXPECT(check_expert_counts(g_err, idx, 8, 8, 256,
                             reinterpret_cast<unsigned long long*>(
                                 reinterpret_cast<char*>(cnt) + 4)),
         MOE_E_INVALID, "misaligned");
}

static void ffn_cases() {
  moe_weights w = int8_experts(256, 2304, 2048);
  const float* x = dev<float>(30);
  const int32_t* rt = dev<int32_t>(31);
  const int32_t* off = dev<int32_t>(32);
  float* rows = dev<float>(33);
  void* ws = dev<void>(34);
  const size_t need = ffn_need(8, 64, 2304, 2048, MOE_W_INT8_ROW);
  EXPECT(check_expert_ffn(g_err, &w, 0, x, 8, rt, off, 64, rows, ws, need), MOE_OK, nullptr);
  EXPECT(check_expert_ffn(g_err, &w, 5, x, 8, rt, off, 64, rows, ws, need), MOE_E_UNSUPPORTED,
         "activation");
  EXPECT(check_expert_ffn(g_err, nullptr, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_INVALID,
         "NULL");
  EXPECT(check_expert_ffn(g_err, &w, 0, x, -2, rt, off, 64, rows, ws, need), MOE_E_INVALID,
         "T=-2");
  EXPECT(check_expert_ffn(g_err, &w, 0, x, 8, rt, nullptr, 64, rows, ws, need), MOE_E_INVALID,
         "offsets");
  EXPECT(check_expert_ffn(g_err, &w, 0, nullptr, 8, rt, off, 64, rows, ws, need), MOE_E_INVALID,
         "x is NULL");
  EXPECT(check_expert_ffn(g_err, &w, 0, x, 8, misaligned<int32_t>(31), off, 64, rows, ws, need),
         MOE_E_INVALID, "aligned");
  EXPECT(check_expert_ffn(g_err, &w, 0, x, 8, rt, off, 64, rows, ws, need - 256),
         MOE_E_WORKSPACE, "too small");
  moe_weights one = int8_experts(1, 2304, 2048);
  EXPECT(check_expert_ffn(g_err, &one, 0, x, 8, nullptr, nullptr, 9, rows, ws, need),
         MOE_E_INVALID, "R_max=9");
  moe_weights bad = w;
  bad.fmt = 9;
  EXPECT(check_expert_ffn(g_err, &bad, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_INVALID,
         "format");
  bad = w;
  bad.d = 16448;
  EXPECT(check_expert_ffn(g_err, &bad, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_UNSUPPORTED,
         "16384");
  bad = w;
  bad.fmt = MOE_W_INT4_B32;
  bad.d = 2304 - 64;  // a multiple of 64 but not of 128
  EXPECT(check_expert_ffn(g_err, &bad, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_UNSUPPORTED,
         "multiples of 128");
  bad = w;
  bad.s_down = nullptr;
  EXPECT(check_expert_ffn(g_err, &bad, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_INVALID,
         "scales");
  bad = w;
  bad.w_down = misaligned<void>(3);
  EXPECT(check_expert_ffn(g_err, &bad, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_INVALID,
         "aligned");
  bad = w;
  bad.fmt = MOE_W_FP32;
  EXPECT(check_expert_ffn(g_err, &bad, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_UNSUPPORTED,
         "tiled");
  bad = w;
  bad.layout = 4;
  EXPECT(check_expert_ffn(g_err, &bad, 0, x, 8, rt, off, 64, rows, ws, need), MOE_E_INVALID,
         "layout");
  EXPECT(check_expert_ffn(g_err, &w, 0, nullptr, 0, nullptr, off, 0, nullptr, nullptr, 0), MOE_OK,
         nullptr);
}

static void forward_cases() {
  moe_layer L = kimi_layer();
  const float* x = dev<float>(40);
  float* y = dev<float>(41);
  void* ws = dev<void>(42);
  const size_t need = fwd_layout(nullptr, &L, 8).bytes;
  EXPECT(check_forward(g_err, "moe_forward", &L, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256), MOE_OK,
         nullptr);
  EXPECT(check_forward(g_err, "moe_forward", &L, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need - 1, 256),
         MOE_E_WORKSPACE, "too small");
  EXPECT(check_forward(g_err, "moe_forward", &L, 3, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_UNSUPPORTED, "activation");
  EXPECT(check_forward(g_err, "moe_forward", &L, 0, x, -1, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "T=-1");
  EXPECT(check_forward(g_err, "moe_forward", &L, 0, x, 8, misaligned<float>(43), y, nullptr, nullptr, ws, need,
                       256),
         MOE_E_INVALID, "aligned");
  EXPECT(check_forward(g_err, "moe_forward", &L, 0, nullptr, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "x is NULL");
  EXPECT(check_forward(g_err, "moe_forward", nullptr, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "layer is NULL");
  moe_layer b = L;
  b.k = 17;
  EXPECT(check_forward(g_err, "moe_forward", &b, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "k=17");
  b = L;
  b.router = MOE_ROUTER_SOFTMAX;
  EXPECT(check_forward(g_err, "moe_forward", &b, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "bias");
  b = L;
  b.shared.n_experts = 2;
  EXPECT(check_forward(g_err, "moe_forward", &b, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "shared.n_experts");
  b = L;
  b.shared.d = 1024;
  EXPECT(check_forward(g_err, "moe_forward", &b, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "shared.d");
  b = L;
  b.w_router = nullptr;
  EXPECT(check_forward(g_err, "moe_forward", &b, 0, x, 8, nullptr, y, nullptr, nullptr, ws, need, 256),
         MOE_E_INVALID, "w_router");
  // every small-batch shape with k <= 16 fits the join area on 256 CUs
  for (int T = 1; T <= 16; ++T) {
    const size_t nT = fwd_layout(nullptr, &L, T).bytes;
    EXPECT(check_forward(g_err, "moe_forward", &L, 0, x, T, nullptr, y, nullptr, nullptr, ws, nT, 256), MOE_OK,
           nullptr);
  }
  EXPECT(check_forward(g_err, "moe_forward", &L, 0, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                       256),
         MOE_OK, nullptr);
  size_t bytes = 0;
  EXPECT(check_layer_workspace_size(g_err, &L, 8, &bytes), MOE_OK, nullptr);
  EXPECT(check_layer_workspace_size(g_err, &L, 8, nullptr), MOE_E_INVALID, "bytes");
  EXPECT(check_layer_workspace_size(g_err, &L, -8, &bytes), MOE_E_INVALID, "T=-8");
  EXPECT(check_workspace_size(g_err, 8, 8, 256, 2304, 2048, MOE_W_INT8_ROW, &bytes), MOE_OK,
         nullptr);
  EXPECT(check_workspace_size(g_err, 8, 0, 256, 2304, 2048, MOE_W_INT8_ROW, &bytes),
         MOE_E_INVALID, "k=0");
  EXPECT(check_workspace_size(g_err, 8, 8, 256, 2304, 2048, 7, &bytes), MOE_E_INVALID, "format");
  EXPECT(check_workspace_size(g_err, 0x7fffffff, 8, 256, 2304, 2048, 1, &bytes), MOE_E_INVALID,
         "overflows");
}

static void combine_tile_quant_cases() {
  const float* rows = dev<float>(50);
  const int32_t* tr = dev<int32_t>(51);
  const float* w = dev<float>(52);
  float* y = dev<float>(53);
  EXPECT(check_combine(g_err, rows, tr, w, nullptr, nullptr, 8, 8, 2304, y), MOE_OK, nullptr);
  EXPECT(check_combine(g_err, rows, tr, w, nullptr, nullptr, 8, 8, 2302, y), MOE_E_UNSUPPORTED,
         "multiple of 4");
  EXPECT(check_combine(g_err, rows, tr, w, nullptr, nullptr, 8, 17, 2304, y), MOE_E_INVALID,
         "k=17");
  EXPECT(check_combine(g_err, rows, tr, w, nullptr, nullptr, -8, 8, 2304, y), MOE_E_INVALID,
         "T=-8");
  EXPECT(check_combine(g_err, nullptr, tr, w, nullptr, nullptr, 8, 8, 2304, y), MOE_E_INVALID,
         "rows");
  EXPECT(check_combine(g_err, rows, tr, w, misaligned<float>(54), nullptr, 8, 8, 2304, y),
         MOE_E_INVALID, "aligned");

  moe_weights src = int8_experts(4, 256, 128);
  src.layout = MOE_LAYOUT_ROWS;
  void* dgu = dev<void>(60);
  void* ddn = dev<void>(61);
  EXPECT(check_tile_weights(g_err, &src, dgu, ddn), MOE_OK, nullptr);
  EXPECT(check_tile_weights(g_err, &src, const_cast<void*>(src.w_gate_up), ddn), MOE_E_INVALID,
         "overlap");
  EXPECT(check_tile_weights(g_err, &src, dgu, reinterpret_cast<char*>(dgu) + 4096),
         MOE_E_INVALID, "overlap");
  EXPECT(check_tile_weights(g_err, &src, nullptr, ddn), MOE_E_INVALID, "destination");
  moe_weights tiled = src;
  tiled.layout = MOE_LAYOUT_TILED;
  EXPECT(check_tile_weights(g_err, &tiled, dgu, ddn), MOE_E_INVALID, "ROWS");

  const void* fw = dev<void>(70);
  void* codes = dev<void>(71);
  float* sc = dev<float>(72);
  EXPECT(check_quantize(g_err, MOE_W_INT8_ROW, MOE_IN_BF16, fw, 1000, 2304, codes, sc), MOE_OK,
         nullptr);
  EXPECT(check_quantize(g_err, MOE_W_FP32, MOE_IN_BF16, fw, 1000, 2304, codes, sc),
         MOE_E_UNSUPPORTED, "quantizer");
  EXPECT(check_quantize(g_err, MOE_W_INT4_B32, MOE_IN_F32, fw, 1000, 2300, codes, sc),
         MOE_E_UNSUPPORTED, "multiple of 32");
  EXPECT(check_quantize(g_err, MOE_W_INT8_ROW, 3, fw, 1000, 2304, codes, sc), MOE_E_INVALID,
         "input type");
  EXPECT(check_quantize(g_err, MOE_W_INT8_ROW, MOE_IN_F32, fw, -1, 2304, codes, sc),
         MOE_E_INVALID, "negative");
  EXPECT(check_quantize(g_err, MOE_W_INT8_ROW, MOE_IN_F32, fw, 1000, 2304, nullptr, sc),
         MOE_E_INVALID, "codes");
  EXPECT(check_quantize(g_err, MOE_W_INT8_ROW, MOE_IN_F32, fw, 1000, 2304, codes,
                        misaligned<float>(72)),
         MOE_E_INVALID, "aligned");
  EXPECT(check_quantize(g_err, MOE_W_INT8_ROW, MOE_IN_F32, fw, 1LL << 33, 2304, codes, sc),
         MOE_E_UNSUPPORTED, "2^32");
}

static void coverage_cases() {
  const unsigned long long* c = dev<unsigned long long>(91);
  int32_t* keep = dev<int32_t>(92);
  int32_t* n = dev<int32_t>(93);
  EXPECT(check_coverage_set(g_err, c, 256, 0.95, 8, keep, n), MOE_OK, nullptr);
  EXPECT(check_coverage_set(g_err, c, 1024, 0.0, 1, keep, n), MOE_OK, nullptr);
  EXPECT(check_coverage_set(g_err, c, 1, 1.0, 16, keep, n), MOE_OK, nullptr);
  EXPECT(check_coverage_set(g_err, c, 0, 0.95, 8, keep, n), MOE_E_INVALID, "E=0");
  EXPECT(check_coverage_set(g_err, c, 1025, 0.95, 8, keep, n), MOE_E_INVALID, "E=1025");
  EXPECT(check_coverage_set(g_err, c, 256, 1.2, 8, keep, n), MOE_E_INVALID, "cover");
  EXPECT(check_coverage_set(g_err, c, 256, -0.1, 8, keep, n), MOE_E_INVALID, "cover");
  EXPECT(check_coverage_set(g_err, c, 256, 0.0 / 0.0, 8, keep, n), MOE_E_INVALID, "cover");
  EXPECT(check_coverage_set(g_err, c, 256, 0.95, 0, keep, n), MOE_E_INVALID, "k=0");
  EXPECT(check_coverage_set(g_err, nullptr, 256, 0.95, 8, keep, n), MOE_E_INVALID,
         "counts is NULL");
  EXPECT(check_coverage_set(g_err, c, 256, 0.95, 8, keep, nullptr), MOE_E_INVALID,
         "n_keep is NULL");
  EXPECT(check_coverage_set(g_err, c, 256, 0.95, 8, misaligned<int32_t>(94), n), MOE_E_INVALID,
         "aligned");
}

static void chained_cases() {
  moe_layer L = kimi_layer();
  const float* x = dev<float>(100);
  float* x_out = dev<float>(101);
  void* ws = dev<void>(102);
  const size_t need = fwd_layout(nullptr, &L, 1).bytes;
  moe_pending in{dev<float>(103), dev<float>(104), dev<float>(105), dev<float>(106), 1, 8, 2304};
  moe_pending out{};
  EXPECT(check_forward_chained(g_err, &L, 0, x, nullptr, nullptr, 1, &out, nullptr, nullptr, ws,
                               need, 256), MOE_OK, nullptr);
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &in, x_out, 1, &out, nullptr, nullptr, ws,
                               need, 256), MOE_OK, nullptr);
  EXPECT(check_forward_chained(g_err, &L, 0, x, &in, x_out, 1, &out, nullptr, nullptr, ws, need,
                               256), MOE_E_INVALID, "exactly one");
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, nullptr, x_out, 1, &out, nullptr, nullptr,
                               ws, need, 256), MOE_E_INVALID, "exactly one");
  EXPECT(check_forward_chained(g_err, &L, 0, x, nullptr, nullptr, 1, nullptr, nullptr, nullptr, ws,
                               need, 256), MOE_E_INVALID, "out is NULL");
  EXPECT(check_forward_chained(g_err, &L, 0, x, nullptr, nullptr, 17, &out, nullptr, nullptr, ws,
                               fwd_layout(nullptr, &L, 17).bytes, 256),
         MOE_E_UNSUPPORTED, "small-batch");
  moe_layer f = L;  // an fp32 shared expert runs apart: no chaining
  f.shared.fmt = MOE_W_FP32;
  f.shared.layout = MOE_LAYOUT_ROWS;
  f.shared.s_gate_up = nullptr;
  f.shared.s_down = nullptr;
  EXPECT(check_forward_chained(g_err, &f, 0, x, nullptr, nullptr, 1, &out, nullptr, nullptr, ws,
                               fwd_layout(nullptr, &f, 1).bytes, 256),
         MOE_E_UNSUPPORTED, "small-batch");
  moe_pending bad = in;
  bad.T = 2;
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &bad, x_out, 1, &out, nullptr, nullptr, ws,
                               need, 256), MOE_E_INVALID, "in has T=2");
  bad = in;
  bad.k = 17;
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &bad, x_out, 1, &out, nullptr, nullptr, ws,
                               need, 256), MOE_E_INVALID, "k=17");
  bad = in;
  bad.rows = nullptr;
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &bad, x_out, 1, &out, nullptr, nullptr, ws,
                               need, 256), MOE_E_INVALID, "in->rows is NULL");
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &in, nullptr, 1, &out, nullptr, nullptr, ws,
                               need, 256), MOE_E_INVALID, "x_out is NULL");
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &in, misaligned<float>(107), 1, &out,
                               nullptr, nullptr, ws, need, 256), MOE_E_INVALID, "aligned");
  bad = in;
  bad.residual = x_out;  // the sum would overwrite values it still reads
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &bad, x_out, 1, &out, nullptr, nullptr, ws,
                               need, 256), MOE_E_INVALID, "overlaps");
  EXPECT(check_forward_chained(g_err, &L, 0, nullptr, &in, x_out, 1, &out, nullptr, nullptr, ws,
                               need - 1, 256), MOE_E_WORKSPACE, "too small");
}

static void probe_cases() {
  const void* buf = dev<void>(81);
  void* sink = dev<void>(82);
  EXPECT(check_probe_read(g_err, buf, 1 << 20, 0, sink), MOE_OK, nullptr);
  EXPECT(check_probe_read(g_err, buf, 1000, 0, sink), MOE_E_INVALID, "multiple of 16");
  EXPECT(check_probe_read(g_err, buf, 0, 0, sink), MOE_E_INVALID, "bytes=0");
  EXPECT(check_probe_read(g_err, buf, 1 << 20, -1, sink), MOE_E_INVALID, "blocks=-1");
  EXPECT(check_probe_read(g_err, buf, 1 << 20, kProbeMaxBlocks + 1, sink), MOE_E_INVALID,
         "blocks=");
  EXPECT(check_probe_read(g_err, nullptr, 1 << 20, 0, sink), MOE_E_INVALID, "buf is NULL");
  EXPECT(check_probe_read(g_err, misaligned<void>(83), 1 << 20, 0, sink), MOE_E_INVALID,
         "aligned");
  EXPECT(check_probe_mfma(g_err, MOE_PROBE_MFMA_16X16X64, 16, 0, sink), MOE_OK, nullptr);
  EXPECT(check_probe_mfma(g_err, MOE_PROBE_MFMA_32X32X32, 16, 2048, sink), MOE_OK, nullptr);
  EXPECT(check_probe_mfma(g_err, 2, 16, 0, sink), MOE_E_INVALID, "shape");
  EXPECT(check_probe_mfma(g_err, MOE_PROBE_MFMA_16X16X64, 0, 0, sink), MOE_E_INVALID, "iters");
  EXPECT(check_probe_mfma(g_err, MOE_PROBE_MFMA_16X16X64, 16, 0, nullptr), MOE_E_INVALID,
         "sink is NULL");
  EXPECT(check_probe_mfma(g_err, MOE_PROBE_MFMA_16X16X64, 16, 0, misaligned<void>(84)),
         MOE_E_INVALID, "aligned");
}

int main() {
  route_cases();
  probe_cases();
  coverage_cases();
  chained_cases();
  permute_counts_cases();
  ffn_cases();
  forward_cases();
  combine_tile_quant_cases();
  printf("argument checks: %d failures of %d cases\n", g_fail, g_cases);
  return g_fail == 0 ? 0 : 1;
}
