// Top-k gating for gfx950 ("FarSkip-Collective" section 2.1: G(A) = s(A W_R^T), s() a sparse
// selection that activates a subset of the experts).
//
// One 64-lane wavefront per token.  Lane l holds logits e = l, l+64, l+128, ... (coalesced row
// read).  Each of the k selection rounds finds the lane-local best untaken expert, then a 6-step
// butterfly over the wavefront picks the winner under the total order
//     a before b  <=>  logit_a > logit_b, or logit_a == logit_b and index_a < index_b,
// so ties go to the lower expert index and every lane agrees on the winner.  Lane i keeps
// winner i.  A NaN logit is read as -infinity: it ranks below every number, so each round still
// returns an expert index in [0, E) (the ids feed the permutation's histogram and scatter).  Weights: softmax over all E logits (wave max and wave sum), or sigmoid, optionally
// renormalised over the k winners.
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

int launch_topk(const float* logits, int64_t T, int32_t E, int32_t k, int gate, int renorm,
                int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const unsigned grid = unsigned(cdiv(T, 4));
  const int vpl = int(cdiv(E, 64));
  ProfScope prof(MOE_K_TOPK, s);
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
