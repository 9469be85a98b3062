// Shared device helpers and host-side status plumbing for libfarskip_moe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <vector>

#include "../../include/farskip_moe.h"

namespace fsm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- host status -----------------------------------------------------------------------------
int fail(int code, const char* fmt, ...);   // records the message, returns code
int check_launch(const char* what);          // MOE_OK or MOE_ERR_HIP after a launch
void clear_error();

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- bf16 <-> f32 (bf16 stored as uint16_t) ----------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// round to nearest even; inputs are finite by precondition (inf stays inf)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// a 16-byte vector of 8 bf16 unpacked to floats
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
}

// ---- opt-in kernel timing (prof.hip): brackets one launch with timing events on its stream ------
class ProfScope {
 public:
  ProfScope(int kind, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  int kind_;
  hipStream_t s_;
  hipEvent_t a_, b_;
};

// Collects the timing events of every launch made on this thread while it lives (instead of the
// process-wide profiler), for a stack call's moe_stack_stats_t.  A null out records nothing.
// finish() waits for the recorded launches and fills *out.
struct ProfRec {
  int kind;
  hipStream_t s;
  hipEvent_t a, b;   // timing events recorded before and after the launch
};
class StatsScope {
 public:
  StatsScope(moe_stack_stats_t* out, hipStream_t main);
  ~StatsScope();
  StatsScope(const StatsScope&) = delete;
  StatsScope& operator=(const StatsScope&) = delete;
  int finish();

 private:
  moe_stack_stats_t* out_;
  hipStream_t main_;
  std::vector<ProfRec> recs_;
};

// ---- internal launchers (defined in the kernel files) -----------------------------------------
int launch_router_logits(const void* A, const void* W_R, const float* bias, int dtype, int64_t T,
                         int64_t d, int32_t E, float* logits, hipStream_t s);
int launch_topk(const float* logits, int64_t T, int32_t E, int32_t k, int gate, int renorm,
                int32_t* topk_idx, float* topk_w, hipStream_t s);
// logits, then top-k: one fused launch where one router tile holds all of a token's logits
int launch_route(const void* A, const void* W_R, const float* bias, int dtype, int64_t T, int64_t d, int32_t E,
                 int32_t k, int gate, int renorm, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s);
size_t permute_ws_bytes(int64_t T, int32_t E, int32_t k);
// moe_permute with its count arrays in the library's fixed device scratch (no workspace argument)
// register-only MFMA throughput launch (diag.hip): shape 0 = 16x16x32, 1 = 32x32x16 bf16
int launch_mfma_ceiling(int shape, int iters, int blocks, float* out, hipStream_t s);
int launch_permute_noalloc(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                           const int32_t* topk_idx, int32_t* offsets, int32_t* sorted_src, int32_t* dest_row,
                           void* A_perm, hipStream_t s);
int launch_permute(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                   const int32_t* topk_idx, int32_t* offsets, int32_t* sorted_src, int32_t* dest_row,
                   void* A_perm, void* ws, hipStream_t s);
// grouped-product M-tile table (tile_start [G+1], tile_group [max_tiles]) for BM-row tiles
int launch_tile_table(const int32_t* offsets, int G, int BM, int max_tiles, int32_t* tile_start,
                      int32_t* tile_group, hipStream_t s);
size_t swiglu_ws_bytes(int64_t N, int32_t G, int64_t c, int dtype);
// gather != null: row r of the grouped input is X[gather[r] / gather_k], X having x_rows rows.
// mid != null: recorded on s between the gate/up and the down product.
// kinds (optional): the two profiler kinds of its products (default: routed or single-group ones)
int launch_grouped_swiglu(const void* X, const int32_t* offsets, int32_t G, const void* W1,
                          const void* W2, const void* W3, int dtype, int64_t N, int64_t d, int64_t c,
                          void* Y, void* ws, hipStream_t s, const int32_t* gather = nullptr,
                          int32_t gather_k = 1, int64_t x_rows = 0, hipEvent_t mid = nullptr,
                          const int* kinds = nullptr);
// out_x (optional) = cast(out), or cast(out + x_addend) with x_addend [T, d] dtype
int launch_combine(const void* Y, int dtype, const float* w, const int32_t* dest_row, int64_t T,
                   int64_t d, int32_t k, const void* addend, const float* residual, float* out,
                   void* out_x, hipStream_t s, const void* x_addend = nullptr);
// MXFP8 (mx.hip): rows of a bf16 matrix -> E4M3 codes + one E8M0 scale per 32 elements
// backward-pass building blocks (gemm.hip); epi codes of the bf16 product
enum { PRODUCT_PLAIN = 0, PRODUCT_F32 = 2, PRODUCT_UG = 3 };
// PRODUCT_UG: B1/B2 are [n_out, K] per group (the forward's layout, ldb/b_k1/b_ksplit unused);
// PRODUCT_PLAIN / PRODUCT_F32: B is K-major, [K, ldb] per group: rows [0, b_k1) of B1, and with
// b_ksplit > 0 rows k >= b_ksplit from B2 (row k - b_ksplit)
int launch_bf16_product(int epi, const void* X, const int32_t* offsets, const int32_t* ts, const int32_t* grp,
                        int32_t G, const void* B1, const void* B2, int64_t b_stride, int64_t ldb, int64_t b_k1,
                        int64_t b_ksplit, int64_t N, int64_t K, int64_t n_out, void* out, hipStream_t s,
                        const int32_t* gather, int32_t gather_k, int64_t x_rows, int prof_kind);
// backward pass of one MoE sublayer (bwd.hip)
size_t layer_bwd_ws_bytes(const moe_stack_cfg_t& c);
int launch_layer_backward(const moe_layer_desc_t& W, const moe_stack_cfg_t& c, const void* A, const float* logits,
                          const int32_t* idx, const float* topk_w, const int32_t* offsets,
                          const int32_t* sorted_src, const int32_t* dest_row, const void* Y, const float* dOut,
                          const float* dOut_shared, const moe_layer_grads_t& gr, void* ws, hipStream_t s);
size_t stack_bwd_ws_bytes(const moe_stack_cfg_t& c, int32_t L);
int launch_stack_backward(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t& c, int mode,
                          const uint8_t* mask, const float* o0, const float* dOL, float* dO0,
                          const moe_layer_grads_t* grads, void* ws, hipStream_t s);
int launch_mx_quantize(const void* X, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t s);
size_t mx_swiglu_ws_bytes(int64_t N, int32_t G, int64_t c);
// the grouped SwiGLU MLP on MXFP8 operands (gather as in launch_grouped_swiglu); Y in bf16
int launch_grouped_swiglu_mx(const uint8_t* Xq, const uint8_t* Xs, const int32_t* offsets, int32_t G,
                             const uint8_t* W1q, const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s,
                             const uint8_t* W3q, const uint8_t* W3s, int64_t N, int64_t d, int64_t c, void* Y,
                             void* ws, hipStream_t s, const int32_t* gather, int32_t gather_k, int64_t x_rows,
                             int phases, uint8_t* Hq, uint8_t* Hs, hipEvent_t mid = nullptr);
// x = cast(o [+ S]) : the FarSkip layer input from the fp32 residual (and the shared output)
int launch_make_input(const float* o, const void* S, int dtype, int64_t T, int64_t d, void* x,
                      hipStream_t s);
// out = (o + A) + S in float32 (out may alias o; S may be null), and x = cast(out) when x is set
int launch_residual_add(const float* o, const void* A, const void* S, int dtype, int64_t T, int64_t d, float* out,
                        void* x, hipStream_t s);

}  // namespace fsm
