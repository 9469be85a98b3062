// Combine and FarSkip layer-input kernels for gfx950.
//
// Combine ("FarSkip-Collective" section 2.1: the routed expert activations are aggregated and
// summed back per token):
//   out[t] = residual[t] + addend[t] + sum_{i<k} w[t,i] * Y[dest_row[t*k+i]]
// as a per-token gather in float32, slots in order, so the result is deterministic and needs no
// float atomics.  Each thread owns 8 consecutive columns of one token (16-byte bf16 / 32-byte fp32
// vectors); a workgroup of 128 threads covers 1024 columns of one token.  The optional rounded
// copy out_x is a next layer's input: x_{j+1} = o_j when the skip is off, or, with x_addend, the
// FarSkip input of the layer after, x_{j+2} = cast(o_j + S_{j+1}) (partial; outdated without
// x_addend), formed while o_j is in registers instead of being read back.
//
// Layer input (section 3, eqs. (8a)/(8b)): x = cast(o) or x = cast(o + S), the "outdated" and
// "partial" FarSkip inputs built from the float32 residual stream and the shared-expert output.
#include "common.h"

namespace fsm {

constexpr int CB_THR = 128;
constexpr int CB_COLS = CB_THR * 8;

__device__ __forceinline__ void load8(const void* base, int dtype, int64_t off, float* f) {
  if (dtype == MOE_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    unpack8(v, f);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

__device__ __forceinline__ void store8(void* base, int dtype, int64_t off, const float* f) {
  if (dtype == MOE_BF16) {
    uint4 v;
    v.x = pack2(f[0], f[1]);
    v.y = pack2(f[2], f[3]);
    v.z = pack2(f[4], f[5]);
    v.w = pack2(f[6], f[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = v;
  } else {
    float* p = static_cast<float*>(base) + off;
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
}

__global__ __launch_bounds__(CB_THR) void k_combine(const void* __restrict__ Y, int dtype,
                                                    const float* __restrict__ w,
                                                    const int32_t* __restrict__ dest_row, int64_t d, int k,
                                                    int col_blocks, const void* __restrict__ addend,
                                                    const float* residual, float* out, void* out_x,
                                                    const void* __restrict__ x_addend) {
  const int64_t t = blockIdx.x / col_blocks;
  const int64_t col = int64_t(blockIdx.x % col_blocks) * CB_COLS + threadIdx.x * 8;
  if (col >= d) return;
  const int64_t o = t * d + col;
  float acc[8];
  if (residual) {
    const float4 a = *reinterpret_cast<const float4*>(residual + o);
    const float4 b = *reinterpret_cast<const float4*>(residual + o + 4);
    acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
    acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  }
  if (addend) {
    float s[8];
    load8(addend, dtype, o, s);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += s[q];
  }
  for (int i = 0; i < k; ++i) {
    const int64_t r = dest_row[t * k + i];
    const float wi = w[t * k + i];
    float y[8];
    load8(Y, dtype, r * d + col, y);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = fmaf(wi, y[q], acc[q]);
  }
  *reinterpret_cast<float4*>(out + o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(out + o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (out_x && x_addend) {
    float s[8];
    load8(x_addend, dtype, o, s);
#pragma unroll
    for (int q = 0; q < 8; ++q) s[q] += acc[q];
    store8(out_x, dtype, o, s);
  } else if (out_x) {
    store8(out_x, dtype, o, acc);
  }
}

// bf16 combine with k fixed at compile time: every Y row of the token is requested before the
// first is used (KK + 3 independent 16-byte loads in flight per thread), then the slots are
// summed in order, as in k_combine.  Y, residual and out are touched once, so they are loaded and
// stored with the nontemporal hint.
typedef unsigned int cb_u32x4 __attribute__((ext_vector_type(4)));
typedef float cb_f32x4 __attribute__((ext_vector_type(4)));

template <int KK>
__global__ __launch_bounds__(CB_THR) void k_combine_bf16(const uint16_t* __restrict__ Y,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ dest_row, int64_t d,
                                                         int col_blocks, const uint16_t* __restrict__ addend,
                                                         const float* residual, float* out,
                                                         uint16_t* __restrict__ out_x,
                                                         const uint16_t* __restrict__ x_addend) {
  const int64_t t = blockIdx.x / col_blocks;
  const int64_t col = int64_t(blockIdx.x % col_blocks) * CB_COLS + threadIdx.x * 8;
  if (col >= d) return;
  const int64_t o = t * d + col;
  cb_u32x4 yv[KK];
  float wi[KK];
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    const int64_t r = dest_row[t * KK + i];
    wi[i] = w[t * KK + i];
    yv[i] = __builtin_nontemporal_load(reinterpret_cast<const cb_u32x4*>(Y + r * d + col));
  }
  cb_f32x4 ra = {0.f, 0.f, 0.f, 0.f}, rb = {0.f, 0.f, 0.f, 0.f};
  if (residual) {
    ra = __builtin_nontemporal_load(reinterpret_cast<const cb_f32x4*>(residual + o));
    rb = __builtin_nontemporal_load(reinterpret_cast<const cb_f32x4*>(residual + o + 4));
  }
  cb_u32x4 av = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
  if (addend) av = __builtin_nontemporal_load(reinterpret_cast<const cb_u32x4*>(addend + o));
  if (x_addend) xv = __builtin_nontemporal_load(reinterpret_cast<const cb_u32x4*>(x_addend + o));
  float acc[8] = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
  if (addend) {
    float s[8];
    unpack8(make_uint4(av[0], av[1], av[2], av[3]), s);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += s[q];
  }
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    float y[8];
    unpack8(make_uint4(yv[i][0], yv[i][1], yv[i][2], yv[i][3]), y);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = fmaf(wi[i], y[q], acc[q]);
  }
  __builtin_nontemporal_store(cb_f32x4{acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<cb_f32x4*>(out + o));
  __builtin_nontemporal_store(cb_f32x4{acc[4], acc[5], acc[6], acc[7]}, reinterpret_cast<cb_f32x4*>(out + o + 4));
  if (out_x) {
    float x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = acc[q];
    if (x_addend) {
      float s[8];
      unpack8(make_uint4(xv[0], xv[1], xv[2], xv[3]), s);
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] += s[q];
    }
    uint4 v;
    v.x = pack2(x[0], x[1]);
    v.y = pack2(x[2], x[3]);
    v.z = pack2(x[4], x[5]);
    v.w = pack2(x[6], x[7]);
    *reinterpret_cast<uint4*>(out_x + o) = v;
  }
}

__global__ __launch_bounds__(256) void k_make_input(const float* __restrict__ o, const void* __restrict__ S,
                                                    int dtype, int64_t n8, void* __restrict__ x) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t off = i * 8;
  // o and S are not read again by this layer's kernels: nontemporal loads
  const cb_f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const cb_f32x4*>(o + off));
  const cb_f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const cb_f32x4*>(o + off + 4));
  float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  if (S && dtype == MOE_BF16) {
    const cb_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const cb_u32x4*>(static_cast<const uint16_t*>(S) + off));
    float s[8];
    unpack8(make_uint4(v[0], v[1], v[2], v[3]), s);
#pragma unroll
    for (int q = 0; q < 8; ++q) f[q] += s[q];
  } else if (S) {
    float s[8];
    load8(S, dtype, off, s);
#pragma unroll
    for (int q = 0; q < 8; ++q) f[q] += s[q];
  }
  store8(x, dtype, off, f);
}

// out = o + A (+ S) in float32 (out may alias o) and, optionally, x = cast(out): the partial
// residual of the attention + MoE wiring (everything except the routed-expert output) and the next
// attention sub-block's input.  A and S are in the workload dtype; S may be null.  The sums run in
// the order (o + A) + S.
__global__ __launch_bounds__(256) void k_residual_add(const float* o, const void* __restrict__ A,
                                                      const void* __restrict__ S, int dtype, int64_t n8, float* out,
                                                      void* __restrict__ x) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t off = i * 8;
  const cb_f32x4 a = *reinterpret_cast<const cb_f32x4*>(o + off);
  const cb_f32x4 b = *reinterpret_cast<const cb_f32x4*>(o + off + 4);
  float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  float t[8];
  load8(A, dtype, off, t);
#pragma unroll
  for (int q = 0; q < 8; ++q) f[q] += t[q];
  if (S) {
    load8(S, dtype, off, t);
#pragma unroll
    for (int q = 0; q < 8; ++q) f[q] += t[q];
  }
  *reinterpret_cast<cb_f32x4*>(out + off) = cb_f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<cb_f32x4*>(out + off + 4) = cb_f32x4{f[4], f[5], f[6], f[7]};
  if (x) store8(x, dtype, off, f);
}

int launch_residual_add(const float* o, const void* A, const void* S, int dtype, int64_t T, int64_t d, float* out,
                        void* x, hipStream_t s) {
  const int64_t n8 = T * d / 8;
  if (n8 == 0) return MOE_OK;
  ProfScope prof(MOE_K_LAYER_INPUT, s);
  k_residual_add<<<unsigned(cdiv(n8, 256)), 256, 0, s>>>(o, A, S, dtype, n8, out, x);
  return check_launch("residual add");
}

int launch_combine(const void* Y, int dtype, const float* w, const int32_t* dest_row, int64_t T,
                   int64_t d, int32_t k, const void* addend, const float* residual, float* out,
                   void* out_x, hipStream_t s, const void* x_addend) {
  if (T == 0) return MOE_OK;
  const int col_blocks = int(cdiv(d, CB_COLS));
  ProfScope prof(MOE_K_COMBINE, s);
  if (dtype == MOE_BF16 && (k == 8 || k == 6 || k == 1)) {
    const auto* Yb = static_cast<const uint16_t*>(Y);
    const auto* Ab = static_cast<const uint16_t*>(addend);
    auto* Xb = static_cast<uint16_t*>(out_x);
    const auto* XAb = static_cast<const uint16_t*>(x_addend);
    const unsigned grid = unsigned(T * col_blocks);
    if (k == 8)
      k_combine_bf16<8><<<grid, CB_THR, 0, s>>>(Yb, w, dest_row, d, col_blocks, Ab, residual, out, Xb, XAb);
    else if (k == 6)
      k_combine_bf16<6><<<grid, CB_THR, 0, s>>>(Yb, w, dest_row, d, col_blocks, Ab, residual, out, Xb, XAb);
    else
      k_combine_bf16<1><<<grid, CB_THR, 0, s>>>(Yb, w, dest_row, d, col_blocks, Ab, residual, out, Xb, XAb);
    return check_launch("combine");
  }
  k_combine<<<unsigned(T * col_blocks), CB_THR, 0, s>>>(Y, dtype, w, dest_row, d, k, col_blocks, addend,
                                                         residual, out, out_x, x_addend);
  return check_launch("combine");
}

int launch_make_input(const float* o, const void* S, int dtype, int64_t T, int64_t d, void* x,
                      hipStream_t s) {
  const int64_t n8 = T * d / 8;
  if (n8 == 0) return MOE_OK;
  ProfScope prof(MOE_K_LAYER_INPUT, s);
  k_make_input<<<unsigned(cdiv(n8, 256)), 256, 0, s>>>(o, S, dtype, n8, x);
  return check_launch("layer input");
}

}  // namespace fsm
