// extern "C" entry points of libfarskip_moe: argument checks on the host, then kernel launches.
// The FarSkip stack scheduler ("FarSkip-Collective" section 3, eqs. (8a)/(8b), and section 4's
// explicit overlap on a second queue) lives at the end of this file.
#include <stdarg.h>
#include <stdio.h>

#include <string>
#include <vector>

#include "common.h"

namespace fsm {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

namespace {

bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
size_t esize(int dt) { return dt == MOE_BF16 ? 2 : 4; }
constexpr int64_t kMaxRows = 0x7FFFFFFF;

int check_route(const void* A, const void* W_R, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                int gate, const float* logits, const int32_t* idx, const float* w) {
  if ((A == nullptr) != (W_R == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "moe_route: A and W_R must both be set or both be NULL");
  if (T < 0 || T > kMaxRows) return fail(MOE_ERR_INVALID_ARG, "moe_route: T=%lld out of range", (long long)T);
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "moe_route: E=%d must be >= 1", E);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_route: need 1 <= k <= E (k=%d, E=%d)", k, E);
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "moe_route: E=%d > %d", E, MOE_MAX_EXPERTS);
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "moe_route: k=%d > %d", k, MOE_MAX_TOPK);
  if (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: unknown gate %d", gate);
  if (A) {
    if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "moe_route: unknown dtype %d", dtype);
    if (d < 1) return fail(MOE_ERR_INVALID_ARG, "moe_route: d=%lld must be >= 1", (long long)d);
    if (dtype == MOE_BF16 && d % 64 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "moe_route: bf16 needs d %% 64 == 0 (d=%lld)", (long long)d);
  }
  if (T > 0 && (!logits || !idx || !w))
    return fail(MOE_ERR_INVALID_ARG, "moe_route: logits, topk_idx and topk_w are required");
  return MOE_OK;
}

int check_permute(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k, const int32_t* idx,
                  const int32_t* off, const int32_t* src, const int32_t* dest, const void* A_perm,
                  const void* ws, size_t ws_bytes) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_permute: T=%lld < 0", (long long)T);
  if (E < 1 || k < 1) return fail(MOE_ERR_INVALID_ARG, "moe_permute: need E >= 1 and k >= 1");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: E=%d > %d", E, MOE_MAX_EXPERTS);
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: k=%d > %d", k, MOE_MAX_TOPK);
  if (T * int64_t(k) > kMaxRows) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: T*k exceeds 2^31-1");
  if (!off) return fail(MOE_ERR_INVALID_ARG, "moe_permute: expert_offsets is required");
  if (T > 0 && (!idx || !src || !dest))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: topk_idx, sorted_src and dest_row are required");
  if (A_perm) {
    if (!A) return fail(MOE_ERR_INVALID_ARG, "moe_permute: A_perm given without A");
    if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "moe_permute: unknown dtype %d", dtype);
    if (d < 1) return fail(MOE_ERR_INVALID_ARG, "moe_permute: d=%lld must be >= 1", (long long)d);
    if ((d * int64_t(esize(dtype))) % 16 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "moe_permute: row bytes must be a multiple of 16");
  }
  const size_t need = permute_ws_bytes(T, E, k);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_permute: workspace %zu bytes, need %zu", ws_bytes, need);
  return MOE_OK;
}

int check_swiglu(const void* X, const int32_t* off, int32_t G, const void* W1, const void* W2, const void* W3,
                 int dtype, int64_t N, int64_t d, int64_t c, const void* Y, const void* ws, size_t ws_bytes,
                 const char* who) {
  if (G < 1) return fail(MOE_ERR_INVALID_ARG, "%s: G=%d must be >= 1", who, G);
  if (G > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: G=%d > %d", who, G, MOE_MAX_EXPERTS);
  if (N < 0 || N > kMaxRows) return fail(MOE_ERR_INVALID_ARG, "%s: N=%lld out of range", who, (long long)N);
  if (d < 1 || c < 1) return fail(MOE_ERR_INVALID_ARG, "%s: d and c must be >= 1", who);
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", who, dtype);
  if (dtype == MOE_BF16 && (d % 64 != 0 || c % 64 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 needs d %% 64 == 0 and c %% 64 == 0 (d=%lld, c=%lld)", who,
                (long long)d, (long long)c);
  if (!off || !W1 || !W2 || !W3) return fail(MOE_ERR_INVALID_ARG, "%s: offsets and weights are required", who);
  if (N > 0 && (!X || !Y)) return fail(MOE_ERR_INVALID_ARG, "%s: X and Y are required", who);
  if (c * d > (int64_t(1) << 40)) return fail(MOE_ERR_UNSUPPORTED, "%s: c*d too large", who);
  const size_t need = swiglu_ws_bytes(N, G, c, dtype);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
  return MOE_OK;
}

int check_combine(const void* Y, int dtype, const float* w, const int32_t* dest, int64_t T, int64_t d,
                  int32_t k, const float* out) {
  if (T < 0 || T > kMaxRows) return fail(MOE_ERR_INVALID_ARG, "moe_combine: T=%lld out of range", (long long)T);
  if (d < 1 || k < 1) return fail(MOE_ERR_INVALID_ARG, "moe_combine: need d >= 1 and k >= 1");
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "moe_combine: unknown dtype %d", dtype);
  if (d % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "moe_combine: needs d %% 8 == 0 (d=%lld)", (long long)d);
  if (T * int64_t(k) > kMaxRows) return fail(MOE_ERR_UNSUPPORTED, "moe_combine: T*k exceeds 2^31-1");
  if (T > 0 && (!Y || !w || !dest || !out))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: Y, topk_w, dest_row and out are required");
  return MOE_OK;
}

// ---- FarSkip stack workspace ---------------------------------------------------------------------
struct StackWs {
  void* x[2];
  void* S[2];
  float* logits[2];
  int32_t* idx[2];
  float* w[2];
  int32_t* offsets;
  int32_t* sorted_src;
  int32_t* dest_row[2];
  int32_t* shared_off;
  void* perm_ws;
  void* Y[2];
  void* gemm_ws;
  void* shared_ws;
  uint8_t* xq[2];   // MXFP8 stack: codes and scales of the layer inputs
  uint8_t* xs[2];
  void* xa[2];      // attention + MoE stack: the attention sub-blocks' inputs and outputs
  void* A[2];
  void* attn_ws;
};

// mx: the MXFP8 stack's buffers (layer-input codes and scales, the MXFP8 product's workspace) in
// place of the bf16 product's workspace
StackWs carve_stack(void* ws, const moe_stack_cfg_t& c, size_t* total, bool mx = false, int64_t c_attn = 0) {
  const size_t es = esize(c.dtype);
  const size_t T = size_t(c.T), d = size_t(c.d), E = size_t(c.E), k = size_t(c.k);
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base + off;
    off = align_up(off + bytes, 256);
    return p;
  };
  StackWs s{};
  for (int b = 0; b < 2; ++b) {
    s.x[b] = take(T * d * es);
    s.S[b] = c.c_shared ? take(T * d * es) : nullptr;
    s.logits[b] = static_cast<float*>(take(T * E * 4));
    s.idx[b] = static_cast<int32_t*>(take(T * k * 4));
    s.w[b] = static_cast<float*>(take(T * k * 4));
  }
  s.offsets = static_cast<int32_t*>(take((E + 1) * 4));
  s.sorted_src = static_cast<int32_t*>(take(T * k * 4));
  for (int b = 0; b < 2; ++b) s.dest_row[b] = static_cast<int32_t*>(take(T * k * 4));
  s.shared_off = static_cast<int32_t*>(take(2 * 4));
  s.perm_ws = take(permute_ws_bytes(c.T, c.E, c.k));
  for (int b = 0; b < 2; ++b) s.Y[b] = take(T * k * d * es);
  s.gemm_ws = mx ? take(mx_swiglu_ws_bytes(c.T * c.k, c.E, c.c)) : take(swiglu_ws_bytes(c.T * c.k, c.E, c.c, c.dtype));
  s.shared_ws = !c.c_shared ? nullptr
                : mx ? take(mx_swiglu_ws_bytes(c.T, 1, c.c_shared)) : take(swiglu_ws_bytes(c.T, 1, c.c_shared, c.dtype));
  if (mx) {
    for (int b = 0; b < 2; ++b) {
      s.xq[b] = static_cast<uint8_t*>(take(T * d));
      s.xs[b] = static_cast<uint8_t*>(take(T * d / 32));
    }
  }
  if (c_attn > 0) {
    for (int b = 0; b < 2; ++b) {
      s.xa[b] = take(T * d * es);
      s.A[b] = take(T * d * es);
    }
    s.attn_ws = take(swiglu_ws_bytes(c.T, 1, c_attn, c.dtype));
  }
  if (total) *total = off;
  return s;
}

__global__ void k_set_shared_offsets(int32_t* off, int32_t T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
  }
}

// shapes, modes and pointers of a stack call (forward or backward); `who` names the entry point
int check_stack_args(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t* cfg, int mode,
                     const float* o0, const float* oL, const char* who, const moe_layer_mx_t* mx = nullptr) {
  if (!layers || !cfg) return fail(MOE_ERR_INVALID_ARG, "%s: layers and cfg are required", who);
  if (L < 1) return fail(MOE_ERR_INVALID_ARG, "%s: L=%d must be >= 1", who, L);
  if (mode != FARSKIP_NONE && mode != FARSKIP_PARTIAL && mode != FARSKIP_OUTDATED)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown mode %d", who, mode);
  const moe_stack_cfg_t& c = *cfg;
  if (c.T < 1 || c.d < 1 || c.c < 1 || c.c_shared < 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: bad shapes", who);
  if (c.E < 1 || c.k < 1 || c.k > c.E)
    return fail(MOE_ERR_INVALID_ARG, "%s: need 1 <= k <= E (k=%d, E=%d)", who, c.k, c.E);
  if (c.E > MOE_MAX_EXPERTS || c.k > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E or k above the library limits", who);
  if (c.gate != MOE_GATE_SOFTMAX && c.gate != MOE_GATE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown gate %d", who, c.gate);
  if (!dtype_ok(c.dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", who, c.dtype);
  if (c.dtype == MOE_BF16 && c.d % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 needs d %% 64 == 0", who);
  if (c.dtype == MOE_BF16 && (c.c % 64 != 0 || c.c_shared % 64 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 needs c and c_shared multiples of 64", who);
  if (c.d % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: needs d %% 8 == 0", who);
  if (c.T * int64_t(c.k) > kMaxRows) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k too large", who);
  if (c.T * c.d * int64_t(esize(c.dtype)) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: a layer input above 2^31 bytes", who);
  if (!o0 || !oL) return fail(MOE_ERR_INVALID_ARG, "%s: o0 and oL are required", who);
  if (o0 == oL) return fail(MOE_ERR_INVALID_ARG, "%s: oL must not alias o0", who);
  if (mx && c.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: the MXFP8 stack needs bf16 layers", who);
  if (mx && (c.d % 128 != 0 || c.c % 128 != 0 || c.c_shared % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "%s: the MXFP8 stack needs d, c and c_shared multiples of 128", who);
  if (mx && (c.T * c.k * c.c >= (int64_t(1) << 31) || c.T * c.c_shared >= (int64_t(1) << 31)))
    return fail(MOE_ERR_UNSUPPORTED, "%s: T * k * c and T * c_shared must be below 2^31", who);
  for (int j = 0; j < L; ++j) {
    const moe_layer_desc_t& l = layers[j];
    if (!l.W_R || (!mx && (!l.W1 || !l.W2 || !l.W3)))
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d is missing routed weights", who, j);
    if (mx && (!mx[j].W1q || !mx[j].W1s || !mx[j].W2q || !mx[j].W2s || !mx[j].W3q || !mx[j].W3s))
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d is missing MXFP8 expert codes or scales", who, j);
    if (c.c_shared && !mx && (!l.Ws1 || !l.Ws2 || !l.Ws3))
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d is missing shared weights", who, j);
    if (c.c_shared && mx &&
        (!mx[j].Ws1q || !mx[j].Ws1s || !mx[j].Ws2q || !mx[j].Ws2s || !mx[j].Ws3q || !mx[j].Ws3s))
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d is missing MXFP8 shared-expert codes or scales", who, j);
  }
  return MOE_OK;
}

int check_stack(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t* cfg, int mode,
                const float* o0, const float* oL, const void* ws, size_t ws_bytes) {
  if (int rc = check_stack_args(layers, L, cfg, mode, o0, oL, "farskip_stack_forward")) return rc;
  size_t need = 0;
  carve_stack(nullptr, *cfg, &need);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "farskip_stack_forward: workspace %zu bytes, need %zu", ws_bytes, need);
  return MOE_OK;
}

struct Events {
  std::vector<hipEvent_t> ev;
  ~Events() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
  int make(size_t n) {
    ev.reserve(n);
    for (size_t i = 0; i < n; ++i) {
      hipEvent_t e;
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return fail(MOE_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(r));
      ev.push_back(e);
    }
    return MOE_OK;
  }
};

int record(hipEvent_t e, hipStream_t s) {
  const hipError_t r = hipEventRecord(e, s);
  return r == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(r));
}
int wait(hipStream_t s, hipEvent_t e) {
  const hipError_t r = hipStreamWaitEvent(s, e, 0);
  return r == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "hipStreamWaitEvent: %s", hipGetErrorString(r));
}

// Layer j (0-based) of the stack; x_j, its routing, its expert outputs Y_j and S_j live in
// buffers [j % 2].
//   main stream: wait route_j; permute_j; routed gate/up_j, record mid_j; routed down_j (Y_j) --
//                nothing else, so the routed GEMMs of consecutive layers run back to back
//   side stream: [skip off at j-1: combine_{j-1}, which also writes x_j = o_{j-1}];
//                route_j(x_j); wait mid_j; S_j = shared_j(x_j);
//                [skip on at j-1: combine_{j-1}: o_{j-1} = o_{j-2} + S_{j-1} + R_{j-1}, which also
//                writes x_{j+1} = o_{j-1} (+ S_j when partial) if the skip is on at j];
//                skip on at j and no such combine (j = 0, or skip off at j-1): x_{j+1} from o_{j-1}
// With the skip on, x_{j+1} needs neither R_j nor o_j, so layer j's shared expert, layer j-1's
// combine (HBM-bound) and layer j+1's router all run beside layer j's routed GEMMs.  They start once
// layer j's gate/up product is done and run beside its down product: measured on the
// DeepSeek-V3-shaped stack, 1.1% faster than beside the gate/up product, whose tiles share weight
// panels and activation rows in each XCD's L2 and lose more to a second kernel on the same CUs.
// The last combine runs after the loop, and s_main waits for it.
// Buffer reuse: permute_{j+2}, topk_{j+2} and GEMM_{j+2} rewrite what combine_j reads; the main
// stream reaches them only after waiting for route_{j+2}, which the side stream records after
// combine_j.  Forming x_{j+1} (combine_{j-1} or make_input_{j+1}) rewrites x_{j-1}, read by
// gate/up_{j-1}; it follows the wait for mid_j.  Events are recorded before the waits that name
// them are enqueued.  The MXFP8 stack's layer-input codes and scales [j % 2] are written right
// after x_j, on the same stream, and read only by GEMM_j, so they follow x_j's reuse rule.
int stack_forward(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t& c, int mode,
                  const uint8_t* mask, const float* o0, float* oL, void* ws, hipStream_t sm,
                  hipStream_t ss, const moe_layer_mx_t* mx = nullptr) {
  StackWs w = carve_stack(ws, c, nullptr, mx != nullptr);
  // MXFP8 stack: each layer input is quantised on s_side as soon as it is formed (before the
  // router that s_main's permutation waits for)
  auto quantize_input = [&](int b) -> int {
    return mx ? launch_mx_quantize(w.x[b], c.T, c.d, w.xq[b], w.xs[b], ss) : MOE_OK;
  };
  const bool two = sm != ss;
  Events E_route, E_mid, E_gemm, E_end;
  if (two) {
    if (int rc = E_route.make(L)) return rc;
    if (int rc = E_mid.make(L)) return rc;
    if (int rc = E_gemm.make(L)) return rc;
    if (int rc = E_end.make(2)) return rc;
    // The inputs (o0, weights) may still be in flight on s_main: s_side starts behind them.
    if (int rc = record(E_end.ev[0], sm)) return rc;
    if (int rc = wait(ss, E_end.ev[0])) return rc;
  }
  const int64_t N = c.T * c.k;
  auto skip_at = [&](int j) { return mode != FARSKIP_NONE && (mask ? mask[j] != 0 : true); };
  // combine_j on the side stream: o_j = o_{j-1} + S_j + R_j into oL (o_{j-1} is o0 for j = 0, else
  // oL itself), plus x_{j+1} = o_j when layer j has no skip and is not the last
  // With the skip on at j, the combine can also form layer j+2's input from o_j while it is in
  // registers: next_x = cast(o_j + next_add) (next_add = S_{j+1} for partial inputs, null for
  // outdated ones), the same values the layer-input kernel would form from o_j read back.
  auto combine = [&](int j, void* next_x = nullptr, const void* next_add = nullptr) -> int {
    const int b = j & 1;
    if (two)
      if (int rc = wait(ss, E_gemm.ev[j])) return rc;
    void* out_x = (!skip_at(j) && j + 1 < L) ? w.x[b ^ 1] : next_x;
    return launch_combine(w.Y[b], c.dtype, w.w[b], w.dest_row[b], c.T, c.d, c.k, c.c_shared ? w.S[b] : nullptr,
                          j == 0 ? o0 : oL, oL, out_x, ss, (out_x && out_x == next_x) ? next_add : nullptr);
  };
  k_set_shared_offsets<<<1, 64, 0, ss>>>(w.shared_off, int32_t(c.T));
  if (int rc = check_launch("stack setup")) return rc;
  if (int rc = launch_make_input(o0, nullptr, c.dtype, c.T, c.d, w.x[0], ss)) return rc;
  if (int rc = quantize_input(0)) return rc;

  for (int j = 0; j < L; ++j) {
    const moe_layer_desc_t& l = layers[j];
    const int cur = j & 1, nxt = cur ^ 1;
    const bool last = j + 1 == L;
    // side: layer j's router
    if (j > 0 && !skip_at(j - 1)) {
      if (int rc = combine(j - 1)) return rc;   // also forms x_j
      if (int rc = quantize_input(cur)) return rc;
    }
    if (int rc = launch_route(w.x[cur], l.W_R, l.bias, c.dtype, c.T, c.d, c.E, c.k, c.gate, c.renormalize,
                              w.logits[cur], w.idx[cur], w.w[cur], ss))
      return rc;
    // main: layer j's permutation
    if (two) {
      if (int rc = record(E_route.ev[j], ss)) return rc;
      if (int rc = wait(sm, E_route.ev[j])) return rc;
    }
    if (int rc = launch_permute(w.x[cur], c.dtype, c.T, c.d, c.E, c.k, w.idx[cur], w.offsets, w.sorted_src,
                                w.dest_row[cur], nullptr, w.perm_ws, sm))
      return rc;
    // main: layer j's routed GEMMs
    if (mx) {
      const moe_layer_mx_t& q = mx[j];
      if (int rc = launch_grouped_swiglu_mx(w.xq[cur], w.xs[cur], w.offsets, c.E, q.W1q, q.W1s, q.W2q, q.W2s, q.W3q,
                                            q.W3s, N, c.d, c.c, w.Y[cur], w.gemm_ws, sm, w.sorted_src, c.k, c.T, 3,
                                            nullptr, nullptr, two ? E_mid.ev[j] : nullptr))
        return rc;
    } else if (int rc = launch_grouped_swiglu(w.x[cur], w.offsets, c.E, l.W1, l.W2, l.W3, c.dtype, N, c.d, c.c,
                                              w.Y[cur], w.gemm_ws, sm, w.sorted_src, c.k, c.T,
                                              two ? E_mid.ev[j] : nullptr)) {
      return rc;
    }
    if (two)
      if (int rc = record(E_gemm.ev[j], sm)) return rc;
    // side: layer j's shared expert, layer j-1's combine, layer j+1's input
    if (two)
      if (int rc = wait(ss, E_mid.ev[j])) return rc;
    if (c.c_shared && mx) {
      const moe_layer_mx_t& q = mx[j];
      if (int rc = launch_grouped_swiglu_mx(w.xq[cur], w.xs[cur], w.shared_off, 1, q.Ws1q, q.Ws1s, q.Ws2q, q.Ws2s,
                                            q.Ws3q, q.Ws3s, c.T, c.d, c.c_shared, w.S[cur], w.shared_ws, ss,
                                            nullptr, 1, c.T, 3, nullptr, nullptr))
        return rc;
    } else if (c.c_shared) {
      if (int rc = launch_grouped_swiglu(w.x[cur], w.shared_off, 1, l.Ws1, l.Ws2, l.Ws3, c.dtype, c.T, c.d,
                                         c.c_shared, w.S[cur], w.shared_ws, ss))
        return rc;
    }
    // x_{j+1} = o_{j-1} (+ S_j): formed by combine_{j-1} when it runs here, else from o_{j-1} in HBM
    const bool input_next = skip_at(j) && !last;
    const void* add = (mode == FARSKIP_PARTIAL) ? w.S[cur] : nullptr;
    if (j > 0 && skip_at(j - 1)) {
      if (int rc = combine(j - 1, input_next ? w.x[nxt] : nullptr, add)) return rc;
    } else if (input_next) {
      if (int rc = launch_make_input(j == 0 ? o0 : oL, add, c.dtype, c.T, c.d, w.x[nxt], ss)) return rc;
    }
    if (input_next)
      if (int rc = quantize_input(nxt)) return rc;
  }
  if (int rc = combine(L - 1)) return rc;
  if (two) {
    if (int rc = record(E_end.ev[1], ss)) return rc;
    if (int rc = wait(sm, E_end.ev[1])) return rc;
  }
  return MOE_OK;
}

// ---- the attention + MoE stack ----------------------------------------------------------------------
// Section 3's wiring of layers made of an attention sub-block and an MoE sub-block (shared S_j and
// routed R_j experts): mode FARSKIP_PAPER takes the attention input as the partial activation
// (eq. 8b) and the MoE input as the outdated one (eq. 8a),
//     attn-in_j = P_{j-1} = o_{j-2} + attn-out_{j-1} + S_{j-1}     (attn-in_0 = o_0)
//     mlp-in_j  = o_{j-1}                                          (mlp-in_0 = o_0)
//     o_j = o_{j-1} + attn-out_j + S_j + R_j;
// mode FARSKIP_NONE is the standard stream (attn-in_j = o_{j-1}, mlp-in_j = o_{j-1} + attn-out_j).  A
// dense SwiGLU block stands in for each attention sub-block.  The residual is float32; sub-block
// inputs are rounded to cfg.dtype.  Buffers [j % 2]: xm (MoE inputs, the workspace's x), xa / A
// (attention inputs / outputs), S, logits, top-k, dest_row, Y.
//   paper mode, per layer j:
//     side: router_j(xm[j]), top-k_j; record route_j
//     main: wait route_j; permute_j; routed gate/up_j, down_j; record gemm_j -- nothing else
//     side: S_j = shared(xm[j]); P_j = o_{j-1} + A_j + S_j into oL (in place; o_0 for j = 0) and
//           xa[j+1] = cast(P_j); A_{j+1} = attn_{j+1}(xa[j+1]) -- layer j+1's attention runs beside
//           layer j's routed experts, the one-GPU form of the overlap the wiring is for;
//           wait gemm_j; combine_j: oL += sum_i w Y_j (in place), xm[j+1] = cast(o_j)
//   none mode, per layer j: side: A_j = attn_j(xa[j]); P_j = o_{j-1} + A_j into oL, xm[j] =
//     cast(P_j); router_j; main: as above; side: S_j; wait gemm_j; combine_j: oL += S_j +
//     sum_i w Y_j, xa[j+1] = cast(o_j).
// Reuse: xm[j+1] (rewritten by combine_j) was last read by layer j-1's gathered gate/up on main,
// which precedes gemm_j; Y / top-k / dest_row [j % 2] are rewritten by layer j+2's kernels, which
// main reaches only after route_{j+2}, recorded on side after combine_j; oL, xa, A, S and the side
// workspaces are touched by the side stream only.
int attn_stack_forward(const moe_layer_desc_t* layers, const moe_attn_desc_t* attn, int32_t L,
                       const moe_stack_cfg_t& c, int64_t c_attn, int mode, const float* o0, float* oL, void* ws,
                       hipStream_t sm, hipStream_t ss) {
  StackWs w = carve_stack(ws, c, nullptr, false, c_attn);
  const bool two = sm != ss;
  const bool paper = mode == FARSKIP_PAPER;
  static const int kAttnKinds[2] = {MOE_K_ATTN_GATE_UP, MOE_K_ATTN_DOWN};
  Events E_route, E_gemm, E_end;
  if (two) {
    if (int rc = E_route.make(L)) return rc;
    if (int rc = E_gemm.make(L)) return rc;
    if (int rc = E_end.make(2)) return rc;
    if (int rc = record(E_end.ev[0], sm)) return rc;
    if (int rc = wait(ss, E_end.ev[0])) return rc;
  }
  const int64_t N = c.T * c.k;
  auto attention = [&](int j, int b) -> int {
    const moe_attn_desc_t& a = attn[j];
    return launch_grouped_swiglu(w.xa[b], w.shared_off, 1, a.Wa1, a.Wa2, a.Wa3, c.dtype, c.T, c.d, c_attn, w.A[b],
                                 w.attn_ws, ss, nullptr, 1, 0, nullptr, kAttnKinds);
  };
  k_set_shared_offsets<<<1, 64, 0, ss>>>(w.shared_off, int32_t(c.T));
  if (int rc = check_launch("stack setup")) return rc;
  if (int rc = launch_make_input(o0, nullptr, c.dtype, c.T, c.d, w.xa[0], ss)) return rc;
  if (paper) {
    if (int rc = launch_make_input(o0, nullptr, c.dtype, c.T, c.d, w.x[0], ss)) return rc;
    if (int rc = attention(0, 0)) return rc;
  }
  for (int j = 0; j < L; ++j) {
    const moe_layer_desc_t& l = layers[j];
    const int cur = j & 1, nxt = cur ^ 1;
    const bool last = j + 1 == L;
    const float* o_prev = j == 0 ? o0 : oL;
    if (!paper) {   // mlp-in_j = o_{j-1} + A_j
      if (int rc = attention(j, cur)) return rc;
      if (int rc = launch_residual_add(o_prev, w.A[cur], nullptr, c.dtype, c.T, c.d, oL, w.x[cur], ss)) return rc;
    }
    if (int rc = launch_route(w.x[cur], l.W_R, l.bias, c.dtype, c.T, c.d, c.E, c.k, c.gate, c.renormalize,
                              w.logits[cur], w.idx[cur], w.w[cur], ss))
      return rc;
    if (two) {
      if (int rc = record(E_route.ev[j], ss)) return rc;
      if (int rc = wait(sm, E_route.ev[j])) return rc;
    }
    if (int rc = launch_permute(w.x[cur], c.dtype, c.T, c.d, c.E, c.k, w.idx[cur], w.offsets, w.sorted_src,
                                w.dest_row[cur], nullptr, w.perm_ws, sm))
      return rc;
    if (int rc = launch_grouped_swiglu(w.x[cur], w.offsets, c.E, l.W1, l.W2, l.W3, c.dtype, N, c.d, c.c, w.Y[cur],
                                       w.gemm_ws, sm, w.sorted_src, c.k, c.T))
      return rc;
    if (two)
      if (int rc = record(E_gemm.ev[j], sm)) return rc;
    // side, beside the routed experts: the shared experts, and in paper mode the partial stream and
    // the next layer's attention
    if (c.c_shared)
      if (int rc = launch_grouped_swiglu(w.x[cur], w.shared_off, 1, l.Ws1, l.Ws2, l.Ws3, c.dtype, c.T, c.d,
                                         c.c_shared, w.S[cur], w.shared_ws, ss))
        return rc;
    if (paper) {
      if (int rc = launch_residual_add(o_prev, w.A[cur], c.c_shared ? w.S[cur] : nullptr, c.dtype, c.T, c.d, oL,
                                       last ? nullptr : w.xa[nxt], ss))
        return rc;
      if (!last)
        if (int rc = attention(j + 1, nxt)) return rc;
    }
    if (two)
      if (int rc = wait(ss, E_gemm.ev[j])) return rc;
    const void* add = (!paper && c.c_shared) ? w.S[cur] : nullptr;
    void* out_x = last ? nullptr : (paper ? w.x[nxt] : w.xa[nxt]);
    if (int rc = launch_combine(w.Y[cur], c.dtype, w.w[cur], w.dest_row[cur], c.T, c.d, c.k, add, oL, oL, out_x, ss))
      return rc;
  }
  if (two) {
    if (int rc = record(E_end.ev[1], ss)) return rc;
    if (int rc = wait(sm, E_end.ev[1])) return rc;
  }
  return MOE_OK;
}

// the stack with an optional moe_stack_stats_t: the call's own launches are timed and, once they have
// finished, summarised per stream
int stack_forward_stats(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t& c, int mode,
                        const uint8_t* mask, const float* o0, float* oL, void* ws, hipStream_t sm, hipStream_t ss,
                        const moe_layer_mx_t* mx, moe_stack_stats_t* stats, const char* who) {
  if (stats) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(sm, &st) == hipSuccess && st != hipStreamCaptureStatusNone)
      return fail(MOE_ERR_INVALID_ARG, "%s: stats cannot be measured while s_main is being captured", who);
  }
  StatsScope scope(stats, sm);
  if (int rc = stack_forward(layers, L, c, mode, mask, o0, oL, ws, sm, ss, mx)) return rc;
  return scope.finish();
}

}  // namespace
}  // namespace fsm

using namespace fsm;

namespace fsm {
// diag.hip: the operand-delivery launch behind moe_delivery_probe
int launch_delivery_probe(int hot_pct, int64_t cold_bytes, int iters, int in_flight, int blocks,
                          const void* buf, float* out, uint64_t* clocks, hipStream_t s);
}  // namespace fsm

extern "C" {

int moe_route(const void* A, const void* W_R, const float* bias, int dtype, int64_t T, int64_t d, int32_t E,
              int32_t k, int gate, int renormalize, float* logits, int32_t* topk_idx, float* topk_w,
              void* stream) {
  clear_error();
  if (int rc = check_route(A, W_R, dtype, T, d, E, k, gate, logits, topk_idx, topk_w)) return rc;
  if (T == 0) return MOE_OK;
  const hipStream_t s = as_stream(stream);
  if (A) return launch_route(A, W_R, bias, dtype, T, d, E, k, gate, renormalize, logits, topk_idx, topk_w, s);
  return launch_topk(logits, T, E, k, gate, renormalize, topk_idx, topk_w, s);
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return permute_ws_bytes(T, E, k);
}

int moe_permute(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k, const int32_t* topk_idx,
                int32_t* expert_offsets, int32_t* sorted_src, int32_t* dest_row, void* A_perm, void* ws,
                size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_permute(A, dtype, T, d, E, k, topk_idx, expert_offsets, sorted_src, dest_row, A_perm, ws,
                             ws_bytes))
    return rc;
  return launch_permute(A, dtype, T, d, E, k, topk_idx, expert_offsets, sorted_src, dest_row, A_perm, ws,
                        as_stream(stream));
}

int moe_permute_noalloc(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                        const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_src, int32_t* dest_row,
                        void* A_perm, void* stream) {
  clear_error();
  // the same checks as moe_permute, with the fixed scratch standing in for the workspace
  const size_t need = permute_ws_bytes(T < 0 ? 0 : T, E < 1 ? 1 : E, k < 1 ? 1 : k);
  if (int rc = check_permute(A, dtype, T, d, E, k, topk_idx, expert_offsets, sorted_src, dest_row, A_perm,
                             reinterpret_cast<void*>(uintptr_t(1)), need))
    return rc;
  return launch_permute_noalloc(A, dtype, T, d, E, k, topk_idx, expert_offsets, sorted_src, dest_row, A_perm,
                                as_stream(stream));
}

size_t moe_grouped_swiglu_workspace_bytes(int64_t N, int32_t G, int64_t c, int dtype) {
  if (N < 0 || G < 1 || c < 1 || !dtype_ok(dtype)) return 0;
  return swiglu_ws_bytes(N, G, c, dtype);
}

int moe_grouped_swiglu(const void* X, const int32_t* group_offsets, int32_t G, const void* W1, const void* W2,
                       const void* W3, int dtype, int64_t N, int64_t d, int64_t c, void* Y, void* ws,
                       size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_swiglu(X, group_offsets, G, W1, W2, W3, dtype, N, d, c, Y, ws, ws_bytes,
                            "moe_grouped_swiglu"))
    return rc;
  return launch_grouped_swiglu(X, group_offsets, G, W1, W2, W3, dtype, N, d, c, Y, ws, as_stream(stream));
}

int moe_grouped_swiglu_gathered(const void* X, int64_t T, const int32_t* sorted_src, int32_t k,
                                const int32_t* group_offsets, int32_t G, const void* W1, const void* W2,
                                const void* W3, int dtype, int64_t N, int64_t d, int64_t c, void* Y, void* ws,
                                size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_swiglu(X, group_offsets, G, W1, W2, W3, dtype, N, d, c, Y, ws, ws_bytes,
                            "moe_grouped_swiglu_gathered"))
    return rc;
  if (T < 0 || k < 1) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_swiglu_gathered: need T >= 0 and k >= 1");
  if (N > 0 && (!sorted_src || T == 0))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_swiglu_gathered: sorted_src and T > 0 are required");
  if (T * d * int64_t(esize(dtype)) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu_gathered: X larger than 2^31 bytes");
  return launch_grouped_swiglu(X, group_offsets, G, W1, W2, W3, dtype, N, d, c, Y, ws, as_stream(stream),
                               sorted_src, k, T);
}

int moe_mx_quantize(const void* X, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, void* stream) {
  clear_error();
  if (rows < 0 || K < 0) return fail(MOE_ERR_INVALID_ARG, "moe_mx_quantize: rows and K must be >= 0");
  if (K % 32 != 0) return fail(MOE_ERR_UNSUPPORTED, "moe_mx_quantize: K=%lld is not a multiple of 32", (long long)K);
  if (rows * K > (int64_t(1) << 40)) return fail(MOE_ERR_UNSUPPORTED, "moe_mx_quantize: rows*K too large");
  if (rows * K > 0 && (!X || !codes || !scales))
    return fail(MOE_ERR_INVALID_ARG, "moe_mx_quantize: X, codes and scales are required");
  return launch_mx_quantize(X, rows, K, codes, scales, as_stream(stream));
}

size_t moe_grouped_swiglu_mxfp8_workspace_bytes(int64_t N, int32_t G, int64_t c) {
  if (N < 0 || G < 1 || c < 1) return 0;
  return mx_swiglu_ws_bytes(N, G, c);
}

size_t moe_grouped_mxfp8_phase_workspace_bytes(int64_t N, int32_t G) {
  if (N < 0 || G < 1) return 0;
  return mx_swiglu_ws_bytes(N, G, 0);
}

namespace {
// shared argument checks of the MXFP8 grouped calls; phases as launch_grouped_swiglu_mx
int check_mx(const char* who, int phases, const uint8_t* Xq, const uint8_t* Xs, int64_t x_rows,
             const int32_t* sorted_src, int32_t k, const int32_t* group_offsets, int32_t G, const uint8_t* W1q,
             const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s, const uint8_t* W3q, const uint8_t* W3s,
             int64_t N, int64_t d, int64_t c, const void* Y, const uint8_t* Hq, const uint8_t* Hs, const void* ws,
             size_t ws_bytes) {
  if (G < 1) return fail(MOE_ERR_INVALID_ARG, "%s: G=%d must be >= 1", who, G);
  if (G > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: G=%d > %d", who, G, MOE_MAX_EXPERTS);
  if (N < 0 || N > kMaxRows) return fail(MOE_ERR_INVALID_ARG, "%s: N=%lld out of range", who, (long long)N);
  if (d < 1 || c < 1) return fail(MOE_ERR_INVALID_ARG, "%s: d and c must be >= 1", who);
  if (d % 128 != 0 || c % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: needs d %% 128 == 0 and c %% 128 == 0 (d=%lld, c=%lld)", who,
                (long long)d, (long long)c);
  if (c * d > (int64_t(1) << 40)) return fail(MOE_ERR_UNSUPPORTED, "%s: c*d too large", who);
  if (N * c >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: N * c must be below 2^31", who);
  if (!group_offsets) return fail(MOE_ERR_INVALID_ARG, "%s: group_offsets is required", who);
  if ((phases & 1) && (!W1q || !W1s || !W2q || !W2s))
    return fail(MOE_ERR_INVALID_ARG, "%s: W1 and W2 codes and scales are required", who);
  if ((phases & 2) && (!W3q || !W3s))
    return fail(MOE_ERR_INVALID_ARG, "%s: W3 codes and scales are required", who);
  if (N > 0 && (phases & 1) && (!Xq || !Xs)) return fail(MOE_ERR_INVALID_ARG, "%s: Xq and Xs are required", who);
  if (N > 0 && (phases & 2) && !Y) return fail(MOE_ERR_INVALID_ARG, "%s: Y is required", who);
  if (N > 0 && phases != 3 && (!Hq || !Hs)) return fail(MOE_ERR_INVALID_ARG, "%s: Hq and Hs are required", who);
  if (phases & 1) {
    if (sorted_src) {
      if (k < 1) return fail(MOE_ERR_INVALID_ARG, "%s: k=%d must be >= 1 with sorted_src", who, k);
      if (N > 0 && x_rows < 1) return fail(MOE_ERR_INVALID_ARG, "%s: x_rows must be >= 1 with sorted_src", who);
    } else if (x_rows != N) {
      return fail(MOE_ERR_INVALID_ARG, "%s: without sorted_src x_rows (%lld) must equal N (%lld)", who,
                  (long long)x_rows, (long long)N);
    }
    if (x_rows < 0 || x_rows * d >= (int64_t(1) << 31))
      return fail(MOE_ERR_UNSUPPORTED, "%s: x_rows * d must be below 2^31", who);
  }
  const size_t need = mx_swiglu_ws_bytes(N, G, phases == 3 ? c : 0);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
  return MOE_OK;
}
}  // namespace

int moe_grouped_swiglu_mxfp8(const uint8_t* Xq, const uint8_t* Xs, int64_t x_rows, const int32_t* sorted_src,
                             int32_t k, const int32_t* group_offsets, int32_t G, const uint8_t* W1q,
                             const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s, const uint8_t* W3q,
                             const uint8_t* W3s, int64_t N, int64_t d, int64_t c, void* Y, void* ws,
                             size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_mx("moe_grouped_swiglu_mxfp8", 3, Xq, Xs, x_rows, sorted_src, k, group_offsets, G, W1q, W1s,
                        W2q, W2s, W3q, W3s, N, d, c, Y, nullptr, nullptr, ws, ws_bytes))
    return rc;
  return launch_grouped_swiglu_mx(Xq, Xs, group_offsets, G, W1q, W1s, W2q, W2s, W3q, W3s, N, d, c, Y, ws,
                                  as_stream(stream), sorted_src, sorted_src ? k : 1, x_rows, 3, nullptr, nullptr);
}

int moe_grouped_mxfp8_gate_up(const uint8_t* Xq, const uint8_t* Xs, int64_t x_rows, const int32_t* sorted_src,
                              int32_t k, const int32_t* group_offsets, int32_t G, const uint8_t* W1q,
                              const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s, int64_t N, int64_t d,
                              int64_t c, uint8_t* Hq, uint8_t* Hs, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_mx("moe_grouped_mxfp8_gate_up", 1, Xq, Xs, x_rows, sorted_src, k, group_offsets, G, W1q, W1s,
                        W2q, W2s, nullptr, nullptr, N, d, c, nullptr, Hq, Hs, ws, ws_bytes))
    return rc;
  return launch_grouped_swiglu_mx(Xq, Xs, group_offsets, G, W1q, W1s, W2q, W2s, nullptr, nullptr, N, d, c, nullptr,
                                  ws, as_stream(stream), sorted_src, sorted_src ? k : 1, x_rows, 1, Hq, Hs);
}

int moe_grouped_mxfp8_down(const uint8_t* Hq, const uint8_t* Hs, const int32_t* group_offsets, int32_t G,
                           const uint8_t* W3q, const uint8_t* W3s, int64_t N, int64_t c, int64_t d, void* Y, void* ws,
                           size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_mx("moe_grouped_mxfp8_down", 2, nullptr, nullptr, N, nullptr, 1, group_offsets, G, nullptr,
                        nullptr, nullptr, nullptr, W3q, W3s, N, d, c, Y, Hq, Hs, ws, ws_bytes))
    return rc;
  return launch_grouped_swiglu_mx(nullptr, nullptr, group_offsets, G, nullptr, nullptr, nullptr, nullptr, W3q, W3s, N,
                                  d, c, Y, ws, as_stream(stream), nullptr, 1, N, 2, const_cast<uint8_t*>(Hq),
                                  const_cast<uint8_t*>(Hs));
}

int moe_combine(const void* Y, int dtype, const float* topk_w, const int32_t* dest_row, int64_t T, int64_t d,
                int32_t k, const void* addend, const float* residual, float* out, void* out_x, void* stream) {
  clear_error();
  if (int rc = check_combine(Y, dtype, topk_w, dest_row, T, d, k, out)) return rc;
  return launch_combine(Y, dtype, topk_w, dest_row, T, d, k, addend, residual, out, out_x, as_stream(stream));
}

size_t farskip_stack_mxfp8_workspace_bytes(const moe_stack_cfg_t* cfg) {
  if (!cfg || cfg->T < 1 || cfg->d < 1 || cfg->c < 1 || cfg->E < 1 || cfg->k < 1 || cfg->dtype != MOE_BF16)
    return 0;
  size_t total = 0;
  carve_stack(nullptr, *cfg, &total, true);
  return total;
}

int farskip_stack_forward_mxfp8(const moe_layer_desc_t* layers, const moe_layer_mx_t* mx, int32_t L,
                                const moe_stack_cfg_t* cfg, int mode, const uint8_t* skip_mask, const float* o0,
                                float* oL, void* ws, size_t ws_bytes, void* s_main, void* s_side,
                                moe_stack_stats_t* stats) {
  clear_error();
  const char* who = "farskip_stack_forward_mxfp8";
  if (!mx) return fail(MOE_ERR_INVALID_ARG, "%s: mx is required", who);
  if (int rc = check_stack_args(layers, L, cfg, mode, o0, oL, who, mx)) return rc;
  size_t need = 0;
  carve_stack(nullptr, *cfg, &need, true);
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
  return stack_forward_stats(layers, L, *cfg, mode, skip_mask, o0, oL, ws, as_stream(s_main), as_stream(s_side), mx,
                             stats, who);
}

size_t farskip_stack_workspace_bytes(const moe_stack_cfg_t* cfg) {
  if (!cfg || cfg->T < 1 || cfg->d < 1 || cfg->c < 1 || cfg->E < 1 || cfg->k < 1 || !dtype_ok(cfg->dtype))
    return 0;
  size_t total = 0;
  carve_stack(nullptr, *cfg, &total);
  return total;
}

int farskip_stack_forward(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t* cfg, int mode,
                          const uint8_t* skip_mask, const float* o0, float* oL, void* ws, size_t ws_bytes,
                          void* s_main, void* s_side, moe_stack_stats_t* stats) {
  clear_error();
  if (int rc = check_stack(layers, L, cfg, mode, o0, oL, ws, ws_bytes)) return rc;
  return stack_forward_stats(layers, L, *cfg, mode, skip_mask, o0, oL, ws, as_stream(s_main), as_stream(s_side),
                             nullptr, stats, "farskip_stack_forward");
}

size_t farskip_attn_moe_stack_workspace_bytes(const moe_stack_cfg_t* cfg, int64_t c_attn) {
  if (!cfg || cfg->T < 1 || cfg->d < 1 || cfg->c < 1 || cfg->E < 1 || cfg->k < 1 || c_attn < 1 || !dtype_ok(cfg->dtype))
    return 0;
  size_t total = 0;
  carve_stack(nullptr, *cfg, &total, false, c_attn);
  return total;
}

int farskip_attn_moe_stack_forward(const moe_layer_desc_t* layers, const moe_attn_desc_t* attn, int32_t L,
                                   const moe_stack_cfg_t* cfg, int64_t c_attn, int mode, const float* o0, float* oL,
                                   void* ws, size_t ws_bytes, void* s_main, void* s_side, moe_stack_stats_t* stats) {
  clear_error();
  const char* who = "farskip_attn_moe_stack_forward";
  if (mode != FARSKIP_NONE && mode != FARSKIP_PAPER)
    return fail(MOE_ERR_INVALID_ARG, "%s: mode must be FARSKIP_NONE or FARSKIP_PAPER (got %d)", who, mode);
  if (int rc = check_stack_args(layers, L, cfg, FARSKIP_NONE, o0, oL, who)) return rc;
  if (!attn) return fail(MOE_ERR_INVALID_ARG, "%s: attn is required", who);
  if (c_attn < 1) return fail(MOE_ERR_INVALID_ARG, "%s: c_attn=%lld must be >= 1", who, (long long)c_attn);
  if (cfg->dtype == MOE_BF16 && c_attn % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 needs c_attn %% 64 == 0", who);
  for (int j = 0; j < L; ++j)
    if (!attn[j].Wa1 || !attn[j].Wa2 || !attn[j].Wa3)
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d is missing attention weights", who, j);
  size_t need = 0;
  carve_stack(nullptr, *cfg, &need, false, c_attn);
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
  const hipStream_t sm = as_stream(s_main), ss = as_stream(s_side);
  if (stats) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(sm, &st) == hipSuccess && st != hipStreamCaptureStatusNone)
      return fail(MOE_ERR_INVALID_ARG, "%s: stats cannot be measured while s_main is being captured", who);
  }
  StatsScope scope(stats, sm);
  if (int rc = attn_stack_forward(layers, attn, L, *cfg, c_attn, mode, o0, oL, ws, sm, ss)) return rc;
  return scope.finish();
}

size_t moe_layer_backward_workspace_bytes(const moe_stack_cfg_t* cfg) {
  if (!cfg || cfg->T < 1 || cfg->d < 1 || cfg->c < 1 || cfg->E < 1 || cfg->k < 1 || cfg->c_shared < 0) return 0;
  return layer_bwd_ws_bytes(*cfg);
}

int moe_layer_backward(const moe_layer_desc_t* W, const moe_stack_cfg_t* cfg, const void* A, const float* logits,
                       const int32_t* topk_idx, const float* topk_w, const int32_t* expert_offsets,
                       const int32_t* sorted_src, const int32_t* dest_row, const void* Y, const float* dOut,
                       const float* dOut_shared, const moe_layer_grads_t* grads, void* ws, size_t ws_bytes,
                       void* stream) {
  clear_error();
  const char* who = "moe_layer_backward";
  if (!W || !cfg || !grads) return fail(MOE_ERR_INVALID_ARG, "%s: W, cfg and grads are required", who);
  const moe_stack_cfg_t& c = *cfg;
  if (c.T < 1 || c.T > kMaxRows || c.d < 1 || c.c < 1 || c.E < 1 || c.k < 1 || c.c_shared < 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: sizes must be positive", who);
  if (c.k > c.E) return fail(MOE_ERR_INVALID_ARG, "%s: k=%d > E=%d", who, c.k, c.E);
  if (c.E > MOE_MAX_EXPERTS || c.k > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E or k beyond the limits", who);
  if (c.gate != MOE_GATE_SOFTMAX && c.gate != MOE_GATE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown gate %d", who, c.gate);
  if (c.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: only bf16 is implemented", who);
  if (c.d % 64 || c.c % 64 || c.c_shared % 64 || c.E % 8)
    return fail(MOE_ERR_UNSUPPORTED, "%s: needs d, c, c_shared multiples of 64 and E a multiple of 8", who);
  if (c.T * c.k > kMaxRows || c.T * c.d * 2 >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: T*k or T*d too large", who);
  if (!A || !logits || !topk_idx || !topk_w || !expert_offsets || !sorted_src || !dest_row || !Y || !dOut)
    return fail(MOE_ERR_INVALID_ARG, "%s: forward tensors and dOut are required", who);
  if (!W->W_R || !W->W1 || !W->W2 || !W->W3) return fail(MOE_ERR_INVALID_ARG, "%s: routed weights are required", who);
  if (c.c_shared > 0 && (!W->Ws1 || !W->Ws2 || !W->Ws3))
    return fail(MOE_ERR_INVALID_ARG, "%s: shared weights are required with c_shared > 0", who);
  if (!grads->dA || !grads->dW_R || !grads->dW1 || !grads->dW2 || !grads->dW3)
    return fail(MOE_ERR_INVALID_ARG, "%s: dA, dW_R, dW1, dW2 and dW3 are required", who);
  if (c.c_shared > 0 && (!grads->dWs1 || !grads->dWs2 || !grads->dWs3))
    return fail(MOE_ERR_INVALID_ARG, "%s: dWs1, dWs2 and dWs3 are required with c_shared > 0", who);
  const size_t need = layer_bwd_ws_bytes(c);
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
  return launch_layer_backward(*W, c, A, logits, topk_idx, topk_w, expert_offsets, sorted_src, dest_row, Y, dOut,
                               dOut_shared, *grads, ws, as_stream(stream));
}

size_t farskip_stack_backward_workspace_bytes(const moe_stack_cfg_t* cfg, int32_t L) {
  if (!cfg || L < 1 || cfg->T < 1 || cfg->d < 1 || cfg->c < 1 || cfg->E < 1 || cfg->k < 1 || cfg->c_shared < 0)
    return 0;
  return stack_bwd_ws_bytes(*cfg, L);
}

int farskip_stack_backward(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t* cfg, int mode,
                           const uint8_t* skip_mask, const float* o0, const float* dOL, float* dO0,
                           const moe_layer_grads_t* grads, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  const char* who = "farskip_stack_backward";
  if (int rc = check_stack_args(layers, L, cfg, mode, o0, dO0, who)) return rc;
  const moe_stack_cfg_t& c = *cfg;
  if (c.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: only bf16 is implemented", who);
  if (c.E % 8) return fail(MOE_ERR_UNSUPPORTED, "%s: needs E a multiple of 8", who);
  if (!dOL || !grads) return fail(MOE_ERR_INVALID_ARG, "%s: dOL and grads are required", who);
  if (dOL == dO0) return fail(MOE_ERR_INVALID_ARG, "%s: dO0 must not alias dOL", who);
  for (int j = 0; j < L; ++j) {
    const moe_layer_grads_t& g = grads[j];
    if (!g.dW_R || !g.dW1 || !g.dW2 || !g.dW3)
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d needs dW_R, dW1, dW2 and dW3", who, j);
    if (c.c_shared > 0 && (!g.dWs1 || !g.dWs2 || !g.dWs3))
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d needs dWs1, dWs2 and dWs3", who, j);
  }
  const size_t need = stack_bwd_ws_bytes(c, L);
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
  return launch_stack_backward(layers, L, c, mode, skip_mask, o0, dOL, dO0, grads, ws, as_stream(stream));
}

size_t moe_workspace_bytes(int op, int64_t T, int64_t d, int32_t E, int32_t k, int64_t c, int32_t L,
                           int64_t c_shared, int dtype) {
  if (T < 0 || E < 1 || k < 1) return 0;
  moe_stack_cfg_t cfg{};
  cfg.T = T;
  cfg.d = d;
  cfg.c = c;
  cfg.c_shared = c_shared;
  cfg.E = E;
  cfg.k = k;
  cfg.gate = MOE_GATE_SOFTMAX;
  cfg.renormalize = 0;
  cfg.dtype = dtype;
  switch (op) {
    case MOE_OP_PERMUTE: return moe_permute_workspace_bytes(T, E, k);
    case MOE_OP_GROUPED_SWIGLU: return moe_grouped_swiglu_workspace_bytes(T * k, E, c, dtype);
    case MOE_OP_GROUPED_SWIGLU_MXFP8: return moe_grouped_swiglu_mxfp8_workspace_bytes(T * k, E, c);
    case MOE_OP_MXFP8_PHASE: return moe_grouped_mxfp8_phase_workspace_bytes(T * k, E);
    case MOE_OP_STACK: return farskip_stack_workspace_bytes(&cfg);
    case MOE_OP_STACK_MXFP8: return farskip_stack_mxfp8_workspace_bytes(&cfg);
    case MOE_OP_LAYER_BACKWARD: return moe_layer_backward_workspace_bytes(&cfg);
    case MOE_OP_STACK_BACKWARD: return farskip_stack_backward_workspace_bytes(&cfg, L);
    default: return 0;
  }
}

int moe_mfma_ceiling(int shape, int32_t iters, int32_t blocks, float* out, void* stream) {
  if (shape < 0 || shape > 2) return fail(MOE_ERR_INVALID_ARG, "moe_mfma_ceiling: shape must be 0, 1 or 2");
  if (iters < 1 || blocks < 1) return fail(MOE_ERR_INVALID_ARG, "moe_mfma_ceiling: iters and blocks must be >= 1");
  if (!out) return fail(MOE_ERR_INVALID_ARG, "moe_mfma_ceiling: out is null");
  return fsm::launch_mfma_ceiling(shape, iters, blocks, out, static_cast<hipStream_t>(stream));
}

int moe_delivery_probe(int32_t hot_pct, int64_t cold_bytes, int32_t iters, int32_t in_flight, int32_t blocks,
                       const void* buf, int64_t buf_bytes, float* out, uint64_t* clocks, void* stream) {
  if (hot_pct < 0 || hot_pct > 100) return fail(MOE_ERR_INVALID_ARG, "moe_delivery_probe: hot_pct must lie in [0, 100]");
  if (cold_bytes < 128 || cold_bytes % 128) return fail(MOE_ERR_INVALID_ARG, "moe_delivery_probe: cold_bytes must be a positive multiple of 128");
  if (iters < 1 || blocks < 1) return fail(MOE_ERR_INVALID_ARG, "moe_delivery_probe: iters and blocks must be >= 1");
  if (in_flight != 1 && in_flight != 2) return fail(MOE_ERR_INVALID_ARG, "moe_delivery_probe: in_flight must be 1 or 2");
  if (!buf || !out) return fail(MOE_ERR_INVALID_ARG, "moe_delivery_probe: buf or out is null");
  const int64_t need = (int64_t(16) << 20) + int64_t(blocks) * cold_bytes;
  if (need > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_delivery_probe: 16 MiB + blocks * cold_bytes must stay below 2 GiB");
  if (buf_bytes < need) return fail(MOE_ERR_INVALID_ARG, "moe_delivery_probe: buf_bytes < 16 MiB + blocks * cold_bytes");
  return fsm::launch_delivery_probe(hot_pct, cold_bytes, iters, in_flight, blocks, buf, out, clocks,
                                    static_cast<hipStream_t>(stream));
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_version(void) { return "farskip_moe 0.1 (gfx950)"; }

}  // extern "C"
