// Register-only bf16 MFMA throughput: an attainable ceiling for the products' rooflines.
//
// Every wave issues `iters` rounds of independent MFMAs on operands held in registers, with no
// memory traffic inside the loop, so the launch measures the matrix cores alone, at whatever clock
// the chip holds under that load.  The two bf16 shapes a tile kernel can be built on are offered:
// v_mfma_f32_16x16x32_bf16 (16 accumulators of 4 values per lane) and v_mfma_f32_32x32x16_bf16 (8
// accumulators of 16 values per lane); both do 262 144 FLOP per wave and round.  The accumulators
// are issued round-robin, so no MFMA waits for the one just before it in its wave.
#include "common.h"

namespace fsm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int SHAPE>
__global__ __launch_bounds__(512) void k_mfma_ceiling(float* __restrict__ out, int iters, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * float(threadIdx.x + i));
    b[i] = (__bf16)(seed * float(i + 1));
  }
  float s = 0.f;
  if (SHAPE == 0) {
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[j][r];
  }
  out[int64_t(blockIdx.x) * 512 + threadIdx.x] = s;   // keeps the products live
}

}  // namespace

int launch_mfma_ceiling(int shape, int iters, int blocks, float* out, hipStream_t s) {
  if (shape == 0) k_mfma_ceiling<0><<<blocks, 512, 0, s>>>(out, iters, 1e-3f);
  else k_mfma_ceiling<1><<<blocks, 512, 0, s>>>(out, iters, 1e-3f);
  return check_launch("mfma ceiling");
}

}  // namespace fsm
