// Backward pass of one MoE sublayer (bf16 storage, fp32 accumulation).
//
// The gradients of out = S(A) + R(A) ("FarSkip-Collective" section 2.1: the router, the modern MLP,
// Dispatch and Combine, the shared expert) with respect to A and every weight: the chain rule of
// the forward, in reverse.  The three products that give activation gradients (dH = dY W3,
// dX = [dU | dG] [W1; W2], and the router's dlogits W_R) run on the forward's grouped bf16 kernel
// with the weights read as stored (K-major, through transposing LDS reads); U and G are recomputed
// by that kernel's gate/up loads (nothing of the forward beyond its outputs is kept).  The weight
// gradients are products whose reduction runs over each expert's rows: k_gemm_kgroup sums one
// expert's segment per output tile, reading dY, H, [dU | dG] and the dense operands as stored; only
// the gathered layer input is copied, transposed, with each expert's rows padded to 64.
//
//   k_combine_bwd    dY[dest_row[t,i]] = w[t,i] dOut[t] (bf16), dw[t,i] = <dOut[t], Y[dest_row[t,i]]>,
//                    and the bf16 copy of the shared experts' output gradient
//   k_gate_bwd       dlogits from dw through the softmax / sigmoid (and renormalisation) Jacobian
//   k_col_partial    per-expert sums of dlogits (the bias gradient), in two deterministic passes
//   k_swiglu_bwd     dU = dH SiLU(G), dG = dH U SiLU'(G), and H = U SiLU(G) for dW3
//   k_transpose      64 x 64 tiles through LDS, gathering rows and padding segments
//   k_gemm_kgroup    C_g = A[:, seg_g] B[:, seg_g]^T in fp32, per group g of K segments
#include <vector>

#include "common.h"
#include "tile_kit.h"

namespace fsm {

namespace {
__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}
}  // namespace

// ---- Combine backward: one workgroup per token ---------------------------------------------------
__global__ __launch_bounds__(256) void k_combine_bwd(const float* __restrict__ dOut, const uint16_t* __restrict__ Y,
                                                     const float* __restrict__ w, const int32_t* __restrict__ dest,
                                                     int32_t d, int32_t k, uint16_t* __restrict__ dY,
                                                     float* __restrict__ dw, const float* __restrict__ dS,
                                                     uint16_t* __restrict__ dS_b) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const float* g = dOut + t * d;
  for (int i = 0; i < k; ++i) {
    const int64_t r = dest[t * k + i];
    const float wi = w[t * k + i];
    float part = 0.f;
    for (int col = threadIdx.x * 8; col < d; col += 256 * 8) {
      const float4 g0 = *reinterpret_cast<const float4*>(g + col), g1 = *reinterpret_cast<const float4*>(g + col + 4);
      float y[8];
      unpack8(*reinterpret_cast<const uint4*>(Y + r * d + col), y);
      part += g0.x * y[0] + g0.y * y[1] + g0.z * y[2] + g0.w * y[3] + g1.x * y[4] + g1.y * y[5] + g1.z * y[6] +
              g1.w * y[7];
      uint4 o;
      o.x = pack2(wi * g0.x, wi * g0.y);
      o.y = pack2(wi * g0.z, wi * g0.w);
      o.z = pack2(wi * g1.x, wi * g1.y);
      o.w = pack2(wi * g1.z, wi * g1.w);
      *reinterpret_cast<uint4*>(dY + r * d + col) = o;
    }
    const float s = block_sum_256(part, red);
    if (threadIdx.x == 0) dw[t * k + i] = s;
  }
  if (dS_b) {   // bf16 copy of the shared experts' output gradient
    const float* gs = dS + t * d;
    for (int col = threadIdx.x * 8; col < d; col += 256 * 8) {
      const float4 g0 = *reinterpret_cast<const float4*>(gs + col), g1 = *reinterpret_cast<const float4*>(gs + col + 4);
      *reinterpret_cast<uint4*>(dS_b + t * d + col) =
          make_uint4(pack2(g0.x, g0.y), pack2(g0.z, g0.w), pack2(g1.x, g1.y), pack2(g1.z, g1.w));
    }
  }
}

// The same with k fixed at compile time: one pass over the columns serves all k slots (dOut is read
// once), and the k dot products are reduced together.
template <int KK>
__global__ __launch_bounds__(256) void k_combine_bwd_k(const float* __restrict__ dOut, const uint16_t* __restrict__ Y,
                                                       const float* __restrict__ w, const int32_t* __restrict__ dest,
                                                       int32_t d, uint16_t* __restrict__ dY, float* __restrict__ dw,
                                                       const float* __restrict__ dS, uint16_t* __restrict__ dS_b) {
  __shared__ float red[4][KK];
  const int64_t t = blockIdx.x;
  const float* g = dOut + t * d;
  int64_t r[KK];
  float wi[KK], part[KK];
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    r[i] = dest[t * KK + i];
    wi[i] = w[t * KK + i];
    part[i] = 0.f;
  }
  for (int col = threadIdx.x * 8; col < d; col += 256 * 8) {
    const float4 g0 = *reinterpret_cast<const float4*>(g + col), g1 = *reinterpret_cast<const float4*>(g + col + 4);
    uint4 yv[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) yv[i] = *reinterpret_cast<const uint4*>(Y + r[i] * d + col);
#pragma unroll
    for (int i = 0; i < KK; ++i) {
      float y[8];
      unpack8(yv[i], y);
      part[i] += g0.x * y[0] + g0.y * y[1] + g0.z * y[2] + g0.w * y[3] + g1.x * y[4] + g1.y * y[5] + g1.z * y[6] +
                 g1.w * y[7];
      *reinterpret_cast<uint4*>(dY + r[i] * d + col) =
          make_uint4(pack2(wi[i] * g0.x, wi[i] * g0.y), pack2(wi[i] * g0.z, wi[i] * g0.w),
                     pack2(wi[i] * g1.x, wi[i] * g1.y), pack2(wi[i] * g1.z, wi[i] * g1.w));
    }
    if (dS_b) {
      const float* gs = dS + t * d;
      const float4 s0 = *reinterpret_cast<const float4*>(gs + col), s1 = *reinterpret_cast<const float4*>(gs + col + 4);
      *reinterpret_cast<uint4*>(dS_b + t * d + col) =
          make_uint4(pack2(s0.x, s0.y), pack2(s0.z, s0.w), pack2(s1.x, s1.y), pack2(s1.z, s1.w));
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    float v = part[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[wave][i] = v;
  }
  __syncthreads();
  if (threadIdx.x < KK) dw[t * KK + threadIdx.x] = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
}

// ---- gate backward: one wave per token ----------------------------------------------------------
// p = softmax(L) over all E (or sigmoid(L)); w_i = p[e_i] (/ P, P = sum of the selected p, when
// renormalising).  dp at the selected experts: dw_i, or (dw_i - sum_m dw_m w_m) / P; then
// softmax: dL_j = p_j (dp_j - sum_a dp_a p_a); sigmoid: dL_j = dp_j p_j (1 - p_j).
__global__ __launch_bounds__(256) void k_gate_bwd(const float* __restrict__ logits, const int32_t* __restrict__ idx,
                                                  const float* __restrict__ dw, int64_t T, int32_t E, int32_t k,
                                                  int gate, int renorm, float* __restrict__ dL,
                                                  uint16_t* __restrict__ dL_b, int32_t ld_b) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* L = logits + t * E;
  float m = -INFINITY, s = 0.f;
  if (gate == MOE_GATE_SOFTMAX) {
    for (int j = lane; j < E; j += 64) m = fmaxf(m, L[j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    for (int j = lane; j < E; j += 64) s += expf(L[j] - m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  }
  auto score = [&](float l) { return gate == MOE_GATE_SOFTMAX ? expf(l - m) / s : 1.f / (1.f + expf(-l)); };
  // per-token scalars over the k selected experts (every lane computes them)
  float P = 0.f, S = 0.f;
  for (int i = 0; i < k; ++i) P += score(L[idx[t * k + i]]);
  for (int i = 0; i < k; ++i) S += dw[t * k + i] * (score(L[idx[t * k + i]]) / P);
  float D = 0.f;   // sum_a dp_a p_a (softmax)
  for (int i = 0; i < k; ++i) {
    const float ps = score(L[idx[t * k + i]]);
    const float dps = renorm ? (dw[t * k + i] - S) / P : dw[t * k + i];
    D += dps * ps;
  }
  for (int j = lane; j < E; j += 64) {
    float dp = 0.f;
    for (int i = 0; i < k; ++i)
      if (idx[t * k + i] == j) dp = renorm ? (dw[t * k + i] - S) / P : dw[t * k + i];
    const float p = score(L[j]);
    const float g = gate == MOE_GATE_SOFTMAX ? p * (dp - D) : dp * p * (1.f - p);
    dL[t * E + j] = g;
    dL_b[t * ld_b + j] = f2bf(g);
  }
  for (int j = E + lane; j < ld_b; j += 64) dL_b[t * ld_b + j] = 0;
}

// ---- column sums of dlogits (bias gradient): partial sums over row chunks, then their sum --------
__global__ __launch_bounds__(256) void k_col_partial(const float* __restrict__ X, int64_t R, int32_t C,
                                                     int64_t rows_per_chunk, float* __restrict__ part) {
  __shared__ float red[4][64];
  const int col = blockIdx.x * 64 + (threadIdx.x & 63), rg = threadIdx.x >> 6;
  const int64_t r0 = int64_t(blockIdx.y) * rows_per_chunk, r1 = min(R, r0 + rows_per_chunk);
  float acc = 0.f;
  if (col < C)
    for (int64_t r = r0 + rg; r < r1; r += 4) acc += X[r * C + col];
  red[rg][threadIdx.x & 63] = acc;
  __syncthreads();
  if (rg == 0 && col < C)
    part[int64_t(blockIdx.y) * C + col] = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
}

__global__ __launch_bounds__(256) void k_col_final(const float* __restrict__ part, int32_t chunks, int32_t C,
                                                   float* __restrict__ out) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= C) return;
  float acc = 0.f;
  for (int c = 0; c < chunks; ++c) acc += part[int64_t(c) * C + col];
  out[col] = acc;
}

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ x, int64_t n, float v) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) x[i] = v;
}

// ---- SwiGLU backward: 8 columns per thread ---------------------------------------------------------
__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint16_t* __restrict__ dH, const uint16_t* __restrict__ UG,
                                                    int64_t rows, int32_t c, uint16_t* __restrict__ DUG,
                                                    uint16_t* __restrict__ H) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;   // chunk of 8 columns
  const int64_t cpr = c / 8;
  if (i >= rows * cpr) return;
  const int64_t r = i / cpr, col = (i - r * cpr) * 8;
  float dh[8], u[8], g[8];
  unpack8(*reinterpret_cast<const uint4*>(dH + r * c + col), dh);
  unpack8(*reinterpret_cast<const uint4*>(UG + r * 2 * c + col), u);
  unpack8(*reinterpret_cast<const uint4*>(UG + r * 2 * c + c + col), g);
  float du[8], dg[8], h[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float sg = 1.f / (1.f + expf(-g[q]));
    const float sl = g[q] * sg;
    du[q] = dh[q] * sl;
    dg[q] = dh[q] * u[q] * (sg * (1.f + g[q] * (1.f - sg)));
    h[q] = u[q] * sl;
  }
  *reinterpret_cast<uint4*>(DUG + r * 2 * c + col) =
      make_uint4(pack2(du[0], du[1]), pack2(du[2], du[3]), pack2(du[4], du[5]), pack2(du[6], du[7]));
  *reinterpret_cast<uint4*>(DUG + r * 2 * c + c + col) =
      make_uint4(pack2(dg[0], dg[1]), pack2(dg[2], dg[3]), pack2(dg[4], dg[5]), pack2(dg[6], dg[7]));
  *reinterpret_cast<uint4*>(H + r * c + col) =
      make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
}

// ---- padded segment offsets: poff[g] = sum_{g' < g} ceil(count_g' / 64) * 64 (one block) --------
__global__ __launch_bounds__(1024) void k_pad_offsets(const int32_t* __restrict__ offsets, int32_t G,
                                                      int32_t* __restrict__ poff) {
  __shared__ int32_t sc[1024];
  const int g = threadIdx.x;
  sc[g] = g < G ? (offsets[g + 1] - offsets[g] + 63) / 64 * 64 : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan
    const int32_t v = g >= o ? sc[g - o] : 0;
    __syncthreads();
    sc[g] += v;
    __syncthreads();
  }
  if (g < G) poff[g + 1] = sc[g];
  if (g == 0) poff[0] = 0;
}

// ---- transpose -----------------------------------------------------------------------------------
// out[c][col0 + j] = X[src(j)][c] for c < C and padded columns j, with src(j) the source row of
// output column j: segmented (offsets / poff given): j in [poff[g], poff[g+1]) maps to row
// offsets[g] + j - poff[g] while that is below offsets[g+1] (zero beyond); plain: row j while
// j < R (zero beyond).  A gathered source reads X row gather[src] / gk.  Batches (blockIdx.z)
// step the input by batch_in and the output by batch_out elements.  C % 8 == 0.
struct TrArgs {
  const uint16_t* X;
  int64_t ldx;
  const int32_t* gather;
  int32_t gk;
  const int32_t* offsets;
  const int32_t* poff;
  int32_t G;
  int64_t R;        // source rows (plain)
  int32_t C;        // source columns = output rows
  uint16_t* out;
  int64_t ldo;
  int64_t col0;
  int64_t batch_in, batch_out;
};

__global__ __launch_bounds__(256) void k_transpose(TrArgs p) {
  __shared__ uint16_t tile[64][72];
  const int tid = threadIdx.x;
  const int64_t j0 = int64_t(blockIdx.x) * 64;
  const int c0 = blockIdx.y * 64;
  const uint16_t* X = p.X + int64_t(blockIdx.z) * p.batch_in;
  uint16_t* out = p.out + int64_t(blockIdx.z) * p.batch_out;
  int64_t rbase = j0, rend = p.R;
  if (p.poff) {
    int lo = 0, hi = p.G;   // the segment g with poff[g] <= j0 < poff[g+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (p.poff[mid] <= j0) lo = mid; else hi = mid;
    }
    rbase = p.offsets[lo] + (j0 - p.poff[lo]);
    rend = p.offsets[lo + 1];
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int q = tid + s * 256, row = q >> 3, ch = q & 7;
    const int64_t r = rbase + row;
    const int col = c0 + ch * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rend && col < p.C) {
      const int64_t src = p.gather ? int64_t(p.gather[r] / p.gk) : r;
      v = *reinterpret_cast<const uint4*>(X + src * p.ldx + col);
    }
    uint16_t* dst = &tile[row][ch * 8];
    dst[0] = uint16_t(v.x); dst[1] = uint16_t(v.x >> 16); dst[2] = uint16_t(v.y); dst[3] = uint16_t(v.y >> 16);
    dst[4] = uint16_t(v.z); dst[5] = uint16_t(v.z >> 16); dst[6] = uint16_t(v.w); dst[7] = uint16_t(v.w >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int q = tid + s * 256, cc = q >> 3, jch = q & 7;
    if (c0 + cc >= p.C) continue;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[jch * 8 + e][cc];
    const uint4 o = make_uint4(uint32_t(v[0]) | (uint32_t(v[1]) << 16), uint32_t(v[2]) | (uint32_t(v[3]) << 16),
                               uint32_t(v[4]) | (uint32_t(v[5]) << 16), uint32_t(v[6]) | (uint32_t(v[7]) << 16));
    *reinterpret_cast<uint4*>(out + int64_t(c0 + cc) * p.ldo + p.col0 + j0 + jch * 8) = o;
  }
}

// ---- K-grouped product -----------------------------------------------------------------------------
// C_g[m][n] = sum over group g's K segment of A[m][k] B[n][k] (fp32 out).  Each operand comes in one
// of two layouts:
//   K-contiguous (a transposed copy): rows [M or N, ld] with K along the row; group g's segment
//     starts at column koff_t[g] (koff_t null: koff[g]) and runs into zero padding up to a
//     multiple of 64;
//   row-major in K ("RM", the activations as the forward keeps them): [K rows, ld], column m (or
//     n); group g's segment is rows [koff[g], koff[g+1]), and rows past it read as zeros (they lie
//     beyond the buffer resource).  Stage rows are 512 bytes with 16-byte chunks XOR-swizzled by
//     2 (row mod 4), and a 16 x 32 fragment is two transposing LDS reads (ds_read_b64_tr_b16).
// The segment of group g holds koff[g+1] - koff[g] K values (koff null: one segment of K).  Output
// rows m < split go to out1 + g * split * N, the rest to out2 + g * (M - split) * N (row m - split).
// 256 x 256 tiles, 8 waves (2 x 4), v_mfma_f32_16x16x32_bf16 with the B fragment first so a lane
// holds four consecutive output columns; two direct-to-LDS stages of 64 K values.
typedef short kg_v4i16 __attribute__((ext_vector_type(4)));
struct KgArgs {
  const uint16_t* A;
  const uint16_t* B;
  float* out1;
  float* out2;
  const int32_t* koff;     // [G+1] segment bounds along K, or null (one segment [0, K))
  const int32_t* koff_t;   // [G+1] segment starts of a K-contiguous operand, or null (= koff)
  int64_t lda, ldb;        // elements per operand row
  int32_t K, M, N, G, split, tm, tn;
};

template <bool ARM, bool BRM>
__global__ __launch_bounds__(512) void k_gemm_kgroup(KgArgs p) {
  constexpr int BM = 256, BN = 256, WAVES_N = 4, BK = 64, RB = BK * 2;   // RB: bytes per K-contiguous LDS row
  constexpr int WTM = 128, WTN = 64, FM = 8, FN = 4, NW = 8, RUN_ROWS = 8;
  constexpr int A_RUNS = BM / RUN_ROWS / NW, B_RUNS = BN / RUN_ROWS / NW;   // 1 KB runs per wave per stage
  constexpr int STAGE = (BM + BN) * BK;   // bf16 elements
  constexpr int AR = ARM ? 2 : 1, BR = BRM ? 2 : 1;   // LDS reads per fragment
  __shared__ __attribute__((aligned(16))) uint16_t s0[STAGE], s1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // workgroup -> tile: each XCD (workgroups b with b % 8 == x) takes one contiguous range of the
  // logical order, so the 32 tiles resident on an XCD at a time are consecutive in it.  Within a
  // group the order goes by blocks of up to 4 M-tiles x 8 N-tiles (M-blocks, then N-blocks within
  // them, then the block's tiles), so those 32 tiles read 4 A panels and 8 B panels between them
  // (81% of their L2 requests can hit) instead of the 2 A and 16 B panels of 2 x 16 tiles.
  const int total = p.G * p.tm * p.tn, b = blockIdx.x;
  const int q8 = total / kXcds, r8 = total % kXcds, x = b % kXcds, i8 = b / kXcds;
  if (i8 >= q8 + (x < r8 ? 1 : 0)) return;
  const int L = x * q8 + min(x, r8) + i8;
  const int g = L / (p.tm * p.tn), rem = L - g * (p.tm * p.tn);
  const int bmb = min(4, p.tm), bnb = min(8, p.tn);
  const int mb = rem / (bmb * p.tn), r2 = rem - mb * bmb * p.tn, mh = min(bmb, p.tm - mb * bmb);
  const int nb = r2 / (mh * bnb), r3 = r2 - nb * mh * bnb, nw = min(bnb, p.tn - nb * bnb);
  const int mt = mb * bmb + r3 / nw, nt = nb * bnb + r3 % nw;
  const int64_t seg0 = p.koff ? p.koff[g] : 0;
  const int K = p.koff ? int(p.koff[g + 1] - seg0) : p.K;
  const int64_t segt = p.koff_t ? p.koff_t[g] : seg0;
  const int m0 = mt * BM, n0 = nt * BN;
  const int mrows = min(BM, p.M - m0), nrows = min(BN, p.N - n0);
  const uint32_t lda = uint32_t(p.lda) * 2u, ldb = uint32_t(p.ldb) * 2u;   // bytes per operand row
  const __amdgpu_buffer_rsrc_t rA = ARM ? make_rsrc(p.A + seg0 * p.lda, int64_t(K) * p.lda * 2)
                                        : make_rsrc(p.A + int64_t(m0) * p.lda + segt, int64_t(mrows) * p.lda * 2);
  const __amdgpu_buffer_rsrc_t rB = BRM ? make_rsrc(p.B + seg0 * p.ldb, int64_t(K) * p.ldb * 2)
                                        : make_rsrc(p.B + int64_t(n0) * p.ldb + segt, int64_t(nrows) * p.ldb * 2);
  // direct-to-LDS: K-contiguous runs are 8 rows of 128 bytes (lane l: row l / 8, chunk (l % 8) ^ row);
  // RM runs are 2 rows of 512 bytes (lane l: row l / 32, chunk (l % 32) ^ 2 (row mod 4))
  const int d_row = lane >> 3, d_ch = (lane & 7) ^ d_row;
  uint32_t dA[A_RUNS], dB[B_RUNS];
#pragma unroll
  for (int i = 0; i < A_RUNS; ++i) {
    if (ARM) {
      const int r = 2 * (wave * A_RUNS + i) + (lane >> 5), lc = (lane & 31) ^ ((2 * r) & 7);
      dA[i] = uint32_t(r) * lda + uint32_t(m0) * 2u + uint32_t(lc) * 16u;
    } else {
      dA[i] = uint32_t((wave * A_RUNS + i) * RUN_ROWS + d_row) * lda + uint32_t(d_ch) * 16u;
    }
  }
#pragma unroll
  for (int i = 0; i < B_RUNS; ++i) {
    if (BRM) {
      const int r = 2 * (wave * B_RUNS + i) + (lane >> 5), lc = (lane & 31) ^ ((2 * r) & 7);
      dB[i] = uint32_t(r) * ldb + uint32_t(n0) * 2u + uint32_t(lc) * 16u;
    } else {
      dB[i] = uint32_t((wave * B_RUNS + i) * RUN_ROWS + d_row) * ldb + uint32_t(d_ch) * 16u;
    }
  }

  // K-contiguous fragment reads: row (base + 16 i + lane % 16), K slice ks: chunk ((4 ks + lane / 16) ^ (lane & 7))
  const int sw = lane & 7, fa0 = (wm * WTM + (lane & 15)) * BK, fb0 = BM * BK + (wn * WTN + (lane & 15)) * BK;
  // RM fragment reads: lane (q = lane / 16, j = lane % 16) reads row 8q + j/4 (+ 4 for its upper K
  // values) at columns 4 (j % 4) .. + 3 of the fragment's 16; those rows' swizzle is 2 (j / 4)
  const int tr_row = (8 * (lane >> 4) + ((lane & 15) >> 2)) * 256 + 4 * (lane & 1);
  const int tr_swz = 2 * ((lane & 15) >> 2);
  const int tr_ca = (wm * WTM) / 8 + ((lane & 3) >> 1), tr_cb = (wn * WTN) / 8 + ((lane & 3) >> 1);
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t kb_zero;
  asm volatile("s_mov_b32 %0, 0" : "=s"(kb_zero));
#define KG_SM(BUF) ((BUF) ? s1 : s0)
#define KG_STAGE(KT, BUF)                                                                        \
  {                                                                                              \
    const uint32_t kba = (ARM ? uint32_t(KT) * BK * lda : uint32_t(KT) * RB) + kb_zero;          \
    const uint32_t kbb = (BRM ? uint32_t(KT) * BK * ldb : uint32_t(KT) * RB) + kb_zero;          \
    _Pragma("unroll") for (int i = 0; i < A_RUNS; ++i)                                           \
      FSM_LDS_DMA16(rA, &KG_SM(BUF)[(wave * A_RUNS + i) * 512], dA[i] + kba);                     \
    _Pragma("unroll") for (int i = 0; i < B_RUNS; ++i)                                           \
      FSM_LDS_DMA16(rB, &KG_SM(BUF)[BM * BK + (wave * B_RUNS + i) * 512], dB[i] + kbb);           \
  }
#define KG_TR(BUF, OFF, KS, CB, H)                                                               \
  __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) kg_v4i16*)(         \
      &KG_SM(BUF)[(OFF) + tr_row + ((KS) * 32 + 4 * (H)) * 256 + (((CB) ^ tr_swz) << 3)]))
#define KG_TRF(BUF, OFF, KS, CB) \
  __builtin_bit_cast(bf16x8, __builtin_shufflevector(KG_TR(BUF, OFF, KS, CB, 0), KG_TR(BUF, OFF, KS, CB, 1), 0, 1, 2, 3, 4, 5, 6, 7))
#define KG_LDA(BUF, KS, I)                                                                       \
  (ARM ? KG_TRF(BUF, 0, KS, tr_ca + 2 * (I))                                                     \
       : *reinterpret_cast<const bf16x8*>(&KG_SM(BUF)[fa0 + (I) * 16 * BK + ((((KS) * 4 + (lane >> 4)) ^ sw) << 3)]))
#define KG_LDB(BUF, KS, J)                                                                       \
  (BRM ? KG_TRF(BUF, BM * BK, KS, tr_cb + 2 * (J))                                               \
       : *reinterpret_cast<const bf16x8*>(&KG_SM(BUF)[fb0 + (J) * 16 * BK + ((((KS) * 4 + (lane >> 4)) ^ sw) << 3)]))
// one stage (two K slices of 32): slice 0's B fragments and first A fragment, then per A row block
// the next A fragment (and, for the first FN blocks, one of slice 1's B fragments) is read before
// the block's FN MFMAs; slice 1 follows with its A fragments read one block ahead.  Scheduling
// groups pin that order so an LDS read is always in flight under FN MFMAs.
#define KG_COMPUTE(BUF)                                                                          \
  {                                                                                              \
    bf16x8 b0[FN], b1[FN], a_cur, a_nxt;                                                         \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) b0[j] = KG_LDB(BUF, 0, j);                    \
    a_cur = KG_LDA(BUF, 0, 0);                                                                   \
    __builtin_amdgcn_sched_group_barrier(0x100, FN * BR + AR, 0);                                \
    _Pragma("unroll") for (int i = 0; i < FN; ++i) {                                             \
      a_nxt = KG_LDA(BUF, 0, i + 1);                                                             \
      b1[i] = KG_LDB(BUF, 1, i);                                                                 \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[j], a_cur, acc[i][j], 0, 0, 0);   \
      __builtin_amdgcn_sched_group_barrier(0x100, AR + BR, 0);                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                        \
      a_cur = a_nxt;                                                                             \
    }                                                                                            \
    _Pragma("unroll") for (int i = FN; i < FM; ++i) {                                            \
      a_nxt = (i + 1 < FM) ? KG_LDA(BUF, 0, i + 1) : KG_LDA(BUF, 1, 0);                          \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[j], a_cur, acc[i][j], 0, 0, 0);   \
      __builtin_amdgcn_sched_group_barrier(0x100, AR, 0);                                        \
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                        \
      a_cur = a_nxt;                                                                             \
    }                                                                                            \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                             \
      if (i + 1 < FM) a_nxt = KG_LDA(BUF, 1, i + 1);                                             \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[j], a_cur, acc[i][j], 0, 0, 0);   \
      if (i + 1 < FM) __builtin_amdgcn_sched_group_barrier(0x100, AR, 0);                        \
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                        \
      a_cur = a_nxt;                                                                             \
    }                                                                                            \
  }
#define KG_BARRIER()                    \
  {                                     \
    asm volatile("" ::: "memory");      \
    __builtin_amdgcn_s_barrier();       \
    asm volatile("" ::: "memory");      \
  }

  const int KT = (K + BK - 1) / BK;   // the last stage's rows past the segment read as zeros
  if (KT == 0) {   // an empty segment: the gradient block is zero (uniform across the workgroup)
    for (int e = tid; e < BM * BN; e += 512) {
      const int m = m0 + e / BN, n = n0 + e % BN;
      if (m < p.M && n < p.N) {
        float* orow = m < p.split ? p.out1 + (int64_t(g) * p.split + m) * p.N
                                  : p.out2 + (int64_t(g) * (p.M - p.split) + (m - p.split)) * p.N;
        orow[n] = 0.f;
      }
    }
    return;
  }
  KG_STAGE(0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  KG_BARRIER();
  for (int kt = 0;;) {
    if (kt + 1 < KT) KG_STAGE(kt + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    KG_COMPUTE(0);
    __builtin_amdgcn_sched_barrier(0);
    if (++kt >= KT) break;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    KG_BARRIER();
    if (kt + 1 < KT) KG_STAGE(kt + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    KG_COMPUTE(1);
    __builtin_amdgcn_sched_barrier(0);
    if (++kt >= KT) break;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    KG_BARRIER();
  }
#undef KG_SM
#undef KG_STAGE
#undef KG_LDA
#undef KG_LDB
#undef KG_TR
#undef KG_TRF
#undef KG_COMPUTE
#undef KG_BARRIER

  // epilogue: lane holds rows m0 + .. + (lane & 15), columns n0 + .. + 4 (lane >> 4) + {0..3}
  const int ml = lane & 15, nl = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WTM + i * 16 + ml;
    if (m >= p.M) continue;
    float* orow = m < p.split ? p.out1 + (int64_t(g) * p.split + m) * p.N
                              : p.out2 + (int64_t(g) * (p.M - p.split) + (m - p.split)) * p.N;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WTN + j * 16 + nl;
      if (n + 3 < p.N) {
        *reinterpret_cast<float4*>(orow + n) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N) orow[n + r] = acc[i][j][r];
      }
    }
  }
}

// ---- host --------------------------------------------------------------------------------------------
namespace {
int64_t r64(int64_t x) { return (x + 63) / 64 * 64; }

struct BwdWs {
  uint16_t *dY, *dOut_b, *dL_b, *UG, *dH, *DUG, *H, *dX, *XT;
  uint16_t *UGs, *dHs, *DUGs, *Hs, *dXs;
  float *dw, *ones, *dLf, *bias_part, *dA_r;
  int32_t *poff, *ts, *grp;
};

constexpr int kBiasChunks = 64;

BwdWs carve_bwd(void* ws, const moe_stack_cfg_t& c, size_t* total) {
  const int64_t T = c.T, d = c.d, cc = c.c, cs = c.c_shared, E = c.E, k = c.k, N = T * k;
  const int64_t Ep = r64(E), Np = r64(N) + 64 * E;
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* q = base + off;
    off = align_up(off + bytes, 256);
    return q;
  };
  auto b16 = [&](int64_t n) { return static_cast<uint16_t*>(take(size_t(n) * 2)); };
  auto f32 = [&](int64_t n) { return static_cast<float*>(take(size_t(n) * 4)); };
  BwdWs w{};
  w.dY = b16(N * d);
  w.dOut_b = b16(T * d);
  w.dw = f32(T * k);
  w.ones = f32(T * k);
  w.dLf = f32(T * E);
  w.dL_b = b16(T * Ep);
  w.bias_part = f32(kBiasChunks * E);
  w.poff = static_cast<int32_t*>(take(size_t(E + 1) * 4));
  w.ts = static_cast<int32_t*>(take(size_t(E + 1) * 4));
  w.grp = static_cast<int32_t*>(take(size_t(cdiv(N, 256) + E) * 4));
  w.UG = b16(N * 2 * cc);
  w.dH = b16(N * cc);
  w.DUG = b16(N * 2 * cc);
  w.H = b16(N * cc);
  w.dX = b16(N * d);
  w.XT = b16(d * Np);
  w.dA_r = f32(T * d);
  if (cs > 0) {
    w.UGs = b16(T * 2 * cs);
    w.dHs = b16(T * cs);
    w.DUGs = b16(T * 2 * cs);
    w.Hs = b16(T * cs);
    w.dXs = b16(T * d);
  }
  if (total) *total = off;
  return w;
}

// transpose of rows [0, R) (or segments) of X [*, ldx] into out [C, ldo] at column col0
int transpose(const uint16_t* X, int64_t ldx, int64_t R, int32_t C, uint16_t* out, int64_t ldo, int64_t col0,
              int64_t out_cols, hipStream_t s, const int32_t* gather = nullptr, int32_t gk = 1,
              const int32_t* offsets = nullptr, const int32_t* poff = nullptr, int32_t G = 0, int batches = 1,
              int64_t batch_in = 0, int64_t batch_out = 0) {
  TrArgs a{X, ldx, gather, gk, offsets, poff, G, R, C, out, ldo, col0, batch_in, batch_out};
  const dim3 grid(unsigned(out_cols / 64), unsigned(cdiv(C, 64)), unsigned(batches));
  ProfScope prof(MOE_K_TRANSPOSE, s);
  k_transpose<<<grid, 256, 0, s>>>(a);
  return check_launch("transpose");
}

// A is row-major in K ([K rows, lda]); B is row-major in K ([K rows, ldb], b_rm) or a K-contiguous
// copy ([N, ldb] with segments at koff_t).  max_rows bounds a segment's rows (32-bit buffer offsets).
int kgroup(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, bool b_rm, const int32_t* koff,
           const int32_t* koff_t, int32_t G, int64_t K, int64_t max_rows, int64_t M, int64_t N, float* out1,
           float* out2, int64_t split, hipStream_t s) {
  if ((max_rows + 64) * lda * 2 >= (int64_t(1) << 31) || (b_rm && (max_rows + 64) * ldb * 2 >= (int64_t(1) << 31)))
    return fail(MOE_ERR_UNSUPPORTED, "weight-gradient product: operand rows above 2^31 bytes");
  KgArgs a{};
  a.A = A; a.B = B; a.out1 = out1; a.out2 = out2 ? out2 : out1; a.koff = koff; a.koff_t = koff_t;
  a.lda = lda; a.ldb = ldb;
  a.K = int32_t(K); a.M = int32_t(M); a.N = int32_t(N); a.G = G; a.split = int32_t(split);
  a.tm = int32_t(cdiv(M, 256)); a.tn = int32_t(cdiv(N, 256));
  const int64_t total = int64_t(G) * a.tm * a.tn;
  ProfScope prof(MOE_K_BWD_WGRAD, s);
  if (b_rm)
    k_gemm_kgroup<true, true><<<dim3(unsigned(total)), 512, 0, s>>>(a);
  else
    k_gemm_kgroup<true, false><<<dim3(unsigned(total)), 512, 0, s>>>(a);
  return check_launch("weight-gradient product");
}
}  // namespace

size_t layer_bwd_ws_bytes(const moe_stack_cfg_t& c) {
  size_t total = 0;
  carve_bwd(nullptr, c, &total);
  return total;
}

#define FSM_TRY(x)       \
  {                      \
    if (int rc_ = (x)) return rc_; \
  }

int launch_layer_backward(const moe_layer_desc_t& W, const moe_stack_cfg_t& c, const void* A, const float* logits,
                          const int32_t* idx, const float* topk_w, const int32_t* offsets,
                          const int32_t* sorted_src, const int32_t* dest_row, const void* Y, const float* dOut,
                          const float* dOut_shared, const moe_layer_grads_t& gr, void* ws, hipStream_t s) {
  const int64_t T = c.T, d = c.d, cc = c.c, cs = c.c_shared, k = c.k, N = T * k;
  const int32_t E = c.E;
  const int64_t Ep = r64(E), Np = r64(N) + 64 * int64_t(E);
  BwdWs w = carve_bwd(ws, c, nullptr);
  const uint16_t* Ab = static_cast<const uint16_t*>(A);

  {  // Combine and gate backward, the bias gradient, unit weights for the final sum
    ProfScope prof(MOE_K_BWD_POINTWISE, s);
    const uint16_t* Yb = static_cast<const uint16_t*>(Y);
    const float* dS = dOut_shared ? dOut_shared : dOut;
    uint16_t* dS_b = cs > 0 ? w.dOut_b : nullptr;
    if (k == 8)
      k_combine_bwd_k<8><<<unsigned(T), 256, 0, s>>>(dOut, Yb, topk_w, dest_row, int32_t(d), w.dY, w.dw, dS, dS_b);
    else if (k == 6)
      k_combine_bwd_k<6><<<unsigned(T), 256, 0, s>>>(dOut, Yb, topk_w, dest_row, int32_t(d), w.dY, w.dw, dS, dS_b);
    else if (k == 4)
      k_combine_bwd_k<4><<<unsigned(T), 256, 0, s>>>(dOut, Yb, topk_w, dest_row, int32_t(d), w.dY, w.dw, dS, dS_b);
    else if (k == 2)
      k_combine_bwd_k<2><<<unsigned(T), 256, 0, s>>>(dOut, Yb, topk_w, dest_row, int32_t(d), w.dY, w.dw, dS, dS_b);
    else if (k == 1)
      k_combine_bwd_k<1><<<unsigned(T), 256, 0, s>>>(dOut, Yb, topk_w, dest_row, int32_t(d), w.dY, w.dw, dS, dS_b);
    else
      k_combine_bwd<<<unsigned(T), 256, 0, s>>>(dOut, Yb, topk_w, dest_row, int32_t(d), int32_t(k), w.dY, w.dw, dS,
                                                dS_b);
    FSM_TRY(check_launch("combine backward"));
    k_gate_bwd<<<unsigned(cdiv(T, 4)), 256, 0, s>>>(logits, idx, w.dw, T, E, int32_t(k), c.gate, c.renormalize,
                                                     w.dLf, w.dL_b, int32_t(Ep));
    FSM_TRY(check_launch("gate backward"));
    if (gr.dbias) {
      const int64_t rpc = cdiv(T, kBiasChunks);
      k_col_partial<<<dim3(unsigned(cdiv(E, 64)), kBiasChunks), 256, 0, s>>>(w.dLf, T, E, rpc, w.bias_part);
      FSM_TRY(check_launch("bias partial sums"));
      k_col_final<<<unsigned(cdiv(E, 256)), 256, 0, s>>>(w.bias_part, kBiasChunks, E, gr.dbias);
      FSM_TRY(check_launch("bias sums"));
    }
    k_fill_f32<<<unsigned(cdiv(T * k, 256)), 256, 0, s>>>(w.ones, T * k, 1.f);
    FSM_TRY(check_launch("fill"));
    k_pad_offsets<<<1, 1024, 0, s>>>(offsets, E, w.poff);
    FSM_TRY(check_launch("padded offsets"));
  }
  FSM_TRY(launch_tile_table(offsets, E, 256, int(cdiv(N, 256) + E), w.ts, w.grp, s));

  // routed experts: recompute U, G; dH = dY W3; dU, dG, H; dX = [dU | dG] [W1; W2]
  // (the products against weights read W3 [d, c] and W1, W2 [c, d] K-major, as stored)
  FSM_TRY(launch_bf16_product(PRODUCT_UG, A, offsets, w.ts, w.grp, E, W.W1, W.W2, cc * d, 0, 0, 0, N, d, cc, w.UG, s,
                              sorted_src, int32_t(k), T, MOE_K_BWD_RECOMPUTE));
  FSM_TRY(launch_bf16_product(PRODUCT_PLAIN, w.dY, offsets, w.ts, w.grp, E, W.W3, nullptr, d * cc, cc, d, 0, N, d, cc,
                              w.dH, s, nullptr, 1, N, MOE_K_BWD_DGRAD));
  {
    ProfScope prof(MOE_K_BWD_POINTWISE, s);
    k_swiglu_bwd<<<unsigned(cdiv(N * (cc / 8), 256)), 256, 0, s>>>(w.dH, w.UG, N, int32_t(cc), w.DUG, w.H);
    FSM_TRY(check_launch("swiglu backward"));
  }
  FSM_TRY(launch_bf16_product(PRODUCT_PLAIN, w.DUG, offsets, w.ts, w.grp, E, W.W1, W.W2, cc * d, d, cc, cc, N, 2 * cc,
                              d, w.dX, s, nullptr, 1, N, MOE_K_BWD_DGRAD));

  // routed weight gradients over each expert's rows: dY, H and [dU | dG] are read as stored; the
  // gathered layer input is copied once, transposed, with each expert's rows padded to 64
  FSM_TRY(transpose(Ab, d, N, int32_t(d), w.XT, Np, 0, Np, s, sorted_src, int32_t(k), offsets, w.poff, E));
  FSM_TRY(kgroup(w.dY, d, w.H, cc, true, offsets, nullptr, E, 0, T, d, cc, gr.dW3, nullptr, d, s));
  FSM_TRY(kgroup(w.DUG, 2 * cc, w.XT, Np, false, offsets, w.poff, E, 0, T, 2 * cc, d, gr.dW1, gr.dW2, cc, s));

  // router: dA_r = dlogits W_R, dW_R = dlogits^T A
  FSM_TRY(launch_bf16_product(PRODUCT_F32, w.dL_b, nullptr, nullptr, nullptr, 1, W.W_R, nullptr, 0, d, E, 0, T, Ep, d,
                              w.dA_r, s, nullptr, 1, T, MOE_K_BWD_DGRAD));
  FSM_TRY(kgroup(w.dL_b, Ep, Ab, d, true, nullptr, nullptr, 1, T, T, E, d, gr.dW_R, nullptr, E, s));

  // shared expert (its output gradient is dOut itself)
  if (cs > 0) {
    FSM_TRY(launch_bf16_product(PRODUCT_UG, A, nullptr, nullptr, nullptr, 1, W.Ws1, W.Ws2, 0, 0, 0, 0, T, d, cs, w.UGs,
                                s, nullptr, 1, T, MOE_K_BWD_RECOMPUTE));
    FSM_TRY(launch_bf16_product(PRODUCT_PLAIN, w.dOut_b, nullptr, nullptr, nullptr, 1, W.Ws3, nullptr, 0, cs, d, 0, T,
                                d, cs, w.dHs, s, nullptr, 1, T, MOE_K_BWD_DGRAD));
    {
      ProfScope prof(MOE_K_BWD_POINTWISE, s);
      k_swiglu_bwd<<<unsigned(cdiv(T * (cs / 8), 256)), 256, 0, s>>>(w.dHs, w.UGs, T, int32_t(cs), w.DUGs, w.Hs);
      FSM_TRY(check_launch("swiglu backward"));
    }
    FSM_TRY(launch_bf16_product(PRODUCT_PLAIN, w.DUGs, nullptr, nullptr, nullptr, 1, W.Ws1, W.Ws2, 0, d, cs, cs, T, 2 * cs,
                                d, w.dXs, s, nullptr, 1, T, MOE_K_BWD_DGRAD));
    FSM_TRY(kgroup(w.dOut_b, d, w.Hs, cs, true, nullptr, nullptr, 1, T, T, d, cs, gr.dWs3, nullptr, d, s));
    FSM_TRY(kgroup(w.DUGs, 2 * cs, Ab, d, true, nullptr, nullptr, 1, T, T, 2 * cs, d, gr.dWs1, gr.dWs2, cs, s));
  }

  // dA[t] = sum over t's slots of dX[dest_row] + the router's and the shared expert's parts
  return launch_combine(w.dX, MOE_BF16, w.ones, dest_row, T, d, int32_t(k), cs > 0 ? w.dXs : nullptr, w.dA_r,
                        gr.dA, nullptr, s);
}
#undef FSM_TRY

// ---- FarSkip stack backward ---------------------------------------------------------------------------
// The stack's forward (section 3: o_j = o_{j-1} + S_j(x_j) + R_j(x_j); x_{j+1} = o_j, or with the
// skip on o_{j-1} + S_j(x_j) (partial, 8b) / o_{j-1} (outdated, 8a)) is replayed on the stream,
// keeping every layer's input, routing and expert outputs; then the layers' backward passes run
// in reverse with the gradients routed along the same graph:
//   dS_j = G_o[j] (+ G_x[j+1] under partial with the skip on), the routed part gets G_o[j];
//   G_o[j-1] += G_o[j]; G_x[j] goes to G_o[j-1] (x_j = o_{j-1}) or G_o[j-2] (x_j skipped o_{j-1}).
// The layer inputs' rounding to bf16 passes the gradient through unchanged.
__global__ __launch_bounds__(256) void k_add_f32(float* __restrict__ y, const float* __restrict__ x, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) y[i] += x[i];
}
__global__ __launch_bounds__(256) void k_sum2_f32(float* __restrict__ z, const float* __restrict__ a,
                                                  const float* __restrict__ b, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) z[i] = a[i] + b[i];
}
__global__ void k_two_offsets(int32_t* off, int32_t T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
  }
}

namespace {
int copy_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
  const hipError_t e = hipMemcpyAsync(dst, src, size_t(n) * 4, hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
}

struct StackBwdWs {
  std::vector<void*> x, Y;
  std::vector<float*> logits, w;
  std::vector<int32_t*> idx, off, src, dest;
  float *o, *dS;
  std::vector<float*> Go, Gx;   // Go[1..L] (Go[0] is the caller's dO0), Gx[1..L]
  void *S, *perm_ws, *gemm_ws, *shared_ws, *layer_ws;
  int32_t* shared_off;
};

StackBwdWs carve_stack_bwd(void* ws, const moe_stack_cfg_t& c, int32_t L, size_t* total) {
  const size_t T = size_t(c.T), d = size_t(c.d), E = size_t(c.E), k = size_t(c.k), N = T * k;
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* q = base + off;
    off = align_up(off + bytes, 256);
    return q;
  };
  StackBwdWs w;
  for (int j = 0; j < L; ++j) {
    w.x.push_back(take(T * d * 2));
    w.logits.push_back(static_cast<float*>(take(T * E * 4)));
    w.idx.push_back(static_cast<int32_t*>(take(T * k * 4)));
    w.w.push_back(static_cast<float*>(take(T * k * 4)));
    w.off.push_back(static_cast<int32_t*>(take((E + 1) * 4)));
    w.src.push_back(static_cast<int32_t*>(take(N * 4)));
    w.dest.push_back(static_cast<int32_t*>(take(N * 4)));
    w.Y.push_back(take(N * d * 2));
  }
  w.o = static_cast<float*>(take(T * d * 4));
  w.dS = static_cast<float*>(take(T * d * 4));
  w.Go.push_back(nullptr);
  w.Gx.push_back(nullptr);
  for (int j = 1; j <= L; ++j) {
    w.Go.push_back(static_cast<float*>(take(T * d * 4)));
    w.Gx.push_back(static_cast<float*>(take(T * d * 4)));
  }
  w.S = c.c_shared ? take(T * d * 2) : nullptr;
  w.perm_ws = take(permute_ws_bytes(c.T, c.E, c.k));
  w.gemm_ws = take(swiglu_ws_bytes(c.T * c.k, c.E, c.c, MOE_BF16));
  w.shared_ws = c.c_shared ? take(swiglu_ws_bytes(c.T, 1, c.c_shared, MOE_BF16)) : nullptr;
  w.shared_off = static_cast<int32_t*>(take(2 * 4));
  w.layer_ws = take(layer_bwd_ws_bytes(c));
  if (total) *total = off;
  return w;
}
}  // namespace

size_t stack_bwd_ws_bytes(const moe_stack_cfg_t& c, int32_t L) {
  size_t total = 0;
  carve_stack_bwd(nullptr, c, L, &total);
  return total;
}

#define FSM_TRY(x)                 \
  {                                \
    if (int rc_ = (x)) return rc_; \
  }

int launch_stack_backward(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t& c, int mode,
                          const uint8_t* mask, const float* o0, const float* dOL, float* dO0,
                          const moe_layer_grads_t* grads, void* ws, hipStream_t s) {
  StackBwdWs w = carve_stack_bwd(ws, c, L, nullptr);
  const int64_t T = c.T, d = c.d, N = c.T * c.k, n = T * d;
  const unsigned blocks = unsigned(cdiv(n, 256));
  auto skip = [&](int j) { return mode != FARSKIP_NONE && (mask ? mask[j] != 0 : true); };   // 0-based layer

  // forward replay (one stream), keeping each layer's input, routing and expert outputs
  k_two_offsets<<<1, 64, 0, s>>>(w.shared_off, int32_t(T));
  FSM_TRY(check_launch("stack setup"));
  FSM_TRY(launch_make_input(o0, nullptr, MOE_BF16, T, d, w.x[0], s));
  const float* o_prev = o0;
  for (int j = 0; j < L; ++j) {
    const moe_layer_desc_t& l = layers[j];
    const bool last = j + 1 == L;
    FSM_TRY(launch_route(w.x[j], l.W_R, l.bias, MOE_BF16, T, d, c.E, c.k, c.gate, c.renormalize, w.logits[j],
                         w.idx[j], w.w[j], s));
    if (c.c_shared)
      FSM_TRY(launch_grouped_swiglu(w.x[j], w.shared_off, 1, l.Ws1, l.Ws2, l.Ws3, MOE_BF16, T, d, c.c_shared, w.S,
                                    w.shared_ws, s));
    if (skip(j) && !last)
      FSM_TRY(launch_make_input(o_prev, mode == FARSKIP_PARTIAL ? w.S : nullptr, MOE_BF16, T, d, w.x[j + 1], s));
    FSM_TRY(launch_permute(w.x[j], MOE_BF16, T, d, c.E, c.k, w.idx[j], w.off[j], w.src[j], w.dest[j], nullptr,
                           w.perm_ws, s));
    FSM_TRY(launch_grouped_swiglu(w.x[j], w.off[j], c.E, l.W1, l.W2, l.W3, MOE_BF16, N, d, c.c, w.Y[j], w.gemm_ws, s,
                                  w.src[j], c.k, T));
    FSM_TRY(launch_combine(w.Y[j], MOE_BF16, w.w[j], w.dest[j], T, d, c.k, c.c_shared ? w.S : nullptr, o_prev, w.o,
                           (!skip(j) && !last) ? w.x[j + 1] : nullptr, s));
    o_prev = w.o;
  }

  // reverse pass: Go[j] = dLoss/do_j (Go[0] is dO0), Gx[j] = dLoss/dx_j
  std::vector<float*> Go(w.Go);
  Go[0] = dO0;
  {
    ProfScope prof(MOE_K_BWD_POINTWISE, s);
    for (int j = 0; j < L; ++j) {
      k_fill_f32<<<blocks, 256, 0, s>>>(Go[j], n, 0.f);
      FSM_TRY(check_launch("fill"));
    }
  }
  FSM_TRY(copy_f32(Go[L], dOL, n, s));
  for (int j = L; j >= 1; --j) {
    const moe_layer_desc_t& l = layers[j - 1];
    const float* dS = Go[j];
    if (mode == FARSKIP_PARTIAL && skip(j - 1) && j < L) {
      ProfScope prof(MOE_K_BWD_POINTWISE, s);
      k_sum2_f32<<<blocks, 256, 0, s>>>(w.dS, Go[j], w.Gx[j + 1], n);
      FSM_TRY(check_launch("sum"));
      dS = w.dS;
    }
    moe_layer_grads_t g = grads[j - 1];
    g.dA = w.Gx[j];
    FSM_TRY(launch_layer_backward(l, c, w.x[j - 1], w.logits[j - 1], w.idx[j - 1], w.w[j - 1], w.off[j - 1],
                                  w.src[j - 1], w.dest[j - 1], w.Y[j - 1], Go[j], dS, g, w.layer_ws, s));
    ProfScope prof(MOE_K_BWD_POINTWISE, s);
    k_add_f32<<<blocks, 256, 0, s>>>(Go[j - 1], Go[j], n);
    float* target = j == 1 ? Go[0] : (!skip(j - 2) ? Go[j - 1] : Go[j - 2]);
    k_add_f32<<<blocks, 256, 0, s>>>(target, w.Gx[j], n);
    FSM_TRY(check_launch("gradient sums"));
    if (grads[j - 1].dA) FSM_TRY(copy_f32(grads[j - 1].dA, w.Gx[j], n, s));
  }
  return MOE_OK;
}
#undef FSM_TRY

}  // namespace fsm
