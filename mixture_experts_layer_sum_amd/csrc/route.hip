// Top-k gating for gfx950 ("FarSkip-Collective" section 2.1: G(A) = s(A W_R^T), s() a sparse
// selection that activates a subset of the experts).
//
// k_topk: one 64-lane wavefront per token (any E up to the library's limit, any k).  Lane l holds
// logits e = l, l+64, l+128, ... (a coalesced row read).  Each of the k selection rounds finds the
// lane-local best untaken expert, then a 6-step butterfly over the wavefront picks the winner under
// the total order
//     a before b  <=>  logit_a > logit_b, or logit_a == logit_b and index_a < index_b,
// so ties go to the lower expert index and every lane agrees on the winner.  Lane i keeps winner i.
// k_topk16 (below) runs the same selection with sixteen lanes per token where E <= 256 and k <= 16.
// A NaN logit is read as -infinity: it ranks below every number, so each round still returns an
// expert index in [0, E) (the ids feed the permutation's histogram and scatter).  Weights: softmax
// over all E logits (row max and row sum), or sigmoid, optionally renormalised over the k winners.
#include "common.h"

namespace fsm {

__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

template <int VPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int64_t T, int E, int k,
                                              int gate, int renorm, int32_t* __restrict__ idx_out,
                                              float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront leaves together
  const float* row = logits + t * E;

  float v[VPL];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = j * 64 + lane;
    if (e < E) {
      const float x = row[e];
      v[j] = x != x ? -INFINITY : x;
    } else {
      v[j] = -INFINITY;
      taken |= 1u << j;
    }
  }

  // softmax statistics over all E logits
  float mx = -INFINITY, sum = 0.f;
  if (gate == MOE_GATE_SOFTMAX) {
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (!(taken >> j & 1u)) mx = fmaxf(mx, v[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (!(taken >> j & 1u)) sum += expf(v[j] - mx);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  }

  float my_v = 0.f;
  int my_e = 0;
  for (int i = 0; i < k; ++i) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = j * 64 + lane;
      if (!(taken >> j & 1u) && better(v[j], e, bv, be)) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == i) {
      my_v = bv;
      my_e = be;
    }
  }

  float w = 0.f;
  if (lane < k) w = (gate == MOE_GATE_SOFTMAX) ? expf(my_v - mx) / sum : 1.0f / (1.0f + expf(-my_v));
  if (renorm) {
    float ws = w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off);
    w = w / ws;
  }
  if (lane < k) {
    idx_out[t * k + lane] = my_e;
    w_out[t * k + lane] = w;
  }
}

// Up to 256 experts and k <= 16: sixteen lanes per token, four tokens per wavefront.  Lane r of a
// token's 16-lane row holds the logits e = r, r + 16, r + 32, ...  Each candidate is one 64-bit key:
// the logit's bits mapped to an unsigned order (the sign-magnitude float order made monotone; -0
// taken as +0, NaN as -infinity) above 0xFFFF - e.  One unsigned maximum therefore picks the larger
// logit and, among equal logits, the lower expert index: the same total order as k_topk.  A row's
// maximum or sum is four DPP row rotations (by 8, 4, 2 and 1 lanes; after them every lane of the row
// holds the result), with no LDS traffic.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key >> 31) ? (key & 0x7FFFFFFFu) : ~key);
}
template <int CTRL>
__device__ __forceinline__ uint32_t row_rot(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint64_t row_max64(uint64_t x) {
#define FSM_ROT_MAX(C)                                                                      \
  {                                                                                         \
    const uint64_t o = (uint64_t(row_rot<C>(uint32_t(x >> 32))) << 32) | row_rot<C>(uint32_t(x)); \
    x = o > x ? o : x;                                                                      \
  }
  FSM_ROT_MAX(0x128) FSM_ROT_MAX(0x124) FSM_ROT_MAX(0x122) FSM_ROT_MAX(0x121)
#undef FSM_ROT_MAX
  return x;
}
__device__ __forceinline__ float row_maxf(float x) {
  x = fmaxf(x, __uint_as_float(row_rot<0x128>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(row_rot<0x124>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(row_rot<0x122>(__float_as_uint(x))));
  return fmaxf(x, __uint_as_float(row_rot<0x121>(__float_as_uint(x))));
}
__device__ __forceinline__ float row_sumf(float x) {
  x += __uint_as_float(row_rot<0x128>(__float_as_uint(x)));
  x += __uint_as_float(row_rot<0x124>(__float_as_uint(x)));
  x += __uint_as_float(row_rot<0x122>(__float_as_uint(x)));
  return x + __uint_as_float(row_rot<0x121>(__float_as_uint(x)));
}

template <int NV>
__global__ __launch_bounds__(256) void k_topk16(const float* __restrict__ logits, int64_t T, int E, int k,
                                                int gate, int renorm, int32_t* __restrict__ idx_out,
                                                float* __restrict__ w_out) {
  const int r = threadIdx.x & 15;
  const int64_t t = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  // rows past the batch run along (the row rotations read every lane of the row) and store nothing
  const bool valid = t < T;
  const float* row = logits + (valid ? t : 0) * int64_t(E);
  float v[NV];
  uint64_t key[NV];   // 0 = no candidate (padding, or already selected)
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = j * 16 + r;
    if (valid && e < E) {
      const float x = row[e];
      v[j] = x != x ? -INFINITY : x;
      key[j] = (uint64_t(order_key(v[j])) << 32) | uint32_t(0xFFFF - e);
    } else {
      v[j] = -INFINITY;
      key[j] = 0;
    }
  }

  // softmax statistics over all E logits
  float mx = -INFINITY, sum = 0.f;
  if (gate == MOE_GATE_SOFTMAX) {
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (key[j]) mx = fmaxf(mx, v[j]);
    mx = row_maxf(mx);
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (key[j]) sum += expf(v[j] - mx);
    sum = row_sumf(sum);
  }

  uint64_t mine = 0;
  for (int i = 0; i < k; ++i) {
    uint64_t b = key[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) b = key[j] > b ? key[j] : b;
    b = row_max64(b);
#pragma unroll
    for (int j = 0; j < NV; ++j) key[j] = key[j] == b ? 0 : key[j];
    if (r == i) mine = b;
  }

  const int my_e = 0xFFFF - int(uint32_t(mine) & 0xFFFFu);
  const float my_v = key_value(uint32_t(mine >> 32));
  float w = 0.f;
  if (r < k) w = (gate == MOE_GATE_SOFTMAX) ? expf(my_v - mx) / sum : 1.0f / (1.0f + expf(-my_v));
  if (renorm) w = w / row_sumf(w);
  if (valid && r < k) {
    idx_out[t * k + r] = my_e;
    w_out[t * k + r] = w;
  }
}

int launch_topk(const float* logits, int64_t T, int32_t E, int32_t k, int gate, int renorm,
                int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (T == 0) return MOE_OK;
  ProfScope prof(MOE_K_TOPK, s);
  if (E <= 256 && k <= 16) {
    const unsigned grid16 = unsigned(cdiv(T, 16));
    const int nv = int(cdiv(E, 16));
    if (nv <= 1) k_topk16<1><<<grid16, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
    else if (nv <= 2) k_topk16<2><<<grid16, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
    else if (nv <= 4) k_topk16<4><<<grid16, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
    else if (nv <= 8) k_topk16<8><<<grid16, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
    else k_topk16<16><<<grid16, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
    return check_launch("top-k");
  }
  const unsigned grid = unsigned(cdiv(T, 4));
  const int vpl = int(cdiv(E, 64));
  if (vpl <= 1) k_topk<1><<<grid, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
  else if (vpl <= 2) k_topk<2><<<grid, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
  else if (vpl <= 4) k_topk<4><<<grid, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
  else if (vpl <= 8) k_topk<8><<<grid, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
  else k_topk<16><<<grid, 256, 0, s>>>(logits, T, E, k, gate, renorm, topk_idx, topk_w);
  return check_launch("top-k");
}

// The route step: router logits, then the top-k kernel on them.  (Selecting inside the router GEMM's
// epilogue, where one 256 x 256 tile holds all of a token's logits, was measured slower for the
// DeepSeek-V3-shaped batch: each CU's one tile then runs 256 rows of cross-lane selection steps
// with eight waves, where this kernel spreads them over thousands of workgroups.)
int launch_route(const void* A, const void* W_R, const float* bias, int dtype, int64_t T, int64_t d, int32_t E,
                 int32_t k, int gate, int renorm, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (int rc = launch_router_logits(A, W_R, bias, dtype, T, d, E, logits, s)) return rc;
  return launch_topk(logits, T, E, k, gate, renorm, topk_idx, topk_w, s);
}

}  // namespace fsm
