// Diagnostics for the products' rooflines: register-only MFMA throughput and operand delivery.
//
// Register-only bf16 MFMA throughput: an attainable ceiling for the products' rooflines.
//
// Every wave issues `iters` rounds of independent MFMAs on operands held in registers, with no
// memory traffic inside the loop, so the launch measures the matrix cores alone, at whatever clock
// the chip holds under that load.  The two bf16 shapes a tile kernel can be built on are offered:
// v_mfma_f32_16x16x32_bf16 (16 accumulators of 4 values per lane) and v_mfma_f32_32x32x16_bf16 (8
// accumulators of 16 values per lane), both 262 144 FLOP per wave and round, and the scaled fp8
// instruction of the MXFP8 products, v_mfma_scale_f32_16x16x128_f8f6f4 (16 accumulators, 1 048 576
// FLOP per wave and round).  The accumulators are issued round-robin, so no MFMA waits for the one
// just before it in its wave.
#include "common.h"
#include "tile_kit.h"

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
  } else if (SHAPE == 2) {
    // scaled fp8: 32 E4M3 codes per lane and operand, unit scales (E8M0 127); 65 536 FLOP per MFMA,
    // so a round of 16 is 1 048 576 FLOP per wave
    typedef int v8i __attribute__((ext_vector_type(8)));
    v8i fa, fb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fa[i] = int(0x38383838u + uint32_t(threadIdx.x & 7) + uint32_t(seed > 1.f));
      fb[i] = int(0x30303030u + uint32_t(i));
    }
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, acc[j], 0, 0, 0, 127, 0, 127);
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

// Operand delivery into LDS, the grouped products' other ceiling.  Each of `blocks` workgroups (one
// per CU: the two 64 KB stages take 128 KB of LDS) runs `iters` stages the way a product's K step
// moves its operands: 8 waves, each stage 64 runs of 1 KB, every lane one 16-byte direct-to-LDS
// buffer load into its run, a wait for the stage, a barrier.  No MFMA.  A run of stage `it` reads
// the hot window (the first 1 MiB of the buffer, which every XCD's L2 keeps) when
// (7 run + 3 it) mod 100 < hot_pct, else the block's own cold region of cold_bytes after the first
// 16 MiB, swept in order (large cold regions stream from HBM, small ones stay in the memory-side
// cache but not in L2).  Over any 100 consecutive stages exactly hot_pct runs of 100 are hot.
// in_flight = 1: the next stage is requested only once the previous one has landed (a two-stage
// product's ring: one stage loads while the other is read); 2: two stages in flight.
template <int IN_FLIGHT>
__global__ __launch_bounds__(512) void k_delivery_probe(const uint8_t* __restrict__ buf, uint32_t records,
                                                        uint32_t cold_bytes, int hot_pct, int iters,
                                                        float* __restrict__ out, uint64_t* __restrict__ clocks) {
  constexpr int NW = 8, PER = 64 / NW, HOT_ROWS = (1 << 20) / 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][65536];
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf, records);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint32_t cold_rows = cold_bytes / 128, cold_base = (16u << 20) + blockIdx.x * cold_bytes;
  uint32_t hrow = (blockIdx.x * 61u) % HOT_ROWS, crow = 0;
  // block 0 times its own loop in shader-clock cycles and in ticks of the 100 MHz constant counter
  const bool timer = clocks && blockIdx.x == 0 && threadIdx.x == 0;
  uint64_t c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    const int st = it & 1;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t run = j * NW + wave, r = run * 8 + (lane >> 3);
      const uint32_t off = int((run * 7u + uint32_t(it) * 3u) % 100u) < hot_pct
                               ? ((hrow + r) % HOT_ROWS) * 128u
                               : cold_base + ((crow + r) % cold_rows) * 128u;
      FSM_LDS_DMA16(rs, &lds[st][run * 1024], off + (lane & 7) * 16u);
    }
    hrow = (hrow + 512) % HOT_ROWS;
    crow = (crow + 512) % cold_rows;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((IN_FLIGHT - 1) * PER));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  if (timer) {
    clocks[0] = __builtin_amdgcn_s_memtime() - c0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  out[int64_t(blockIdx.x) * 512 + threadIdx.x] = float(lds[0][threadIdx.x * 4]) + float(lds[1][threadIdx.x * 4]);
}

}  // namespace

int launch_delivery_probe(int hot_pct, int64_t cold_bytes, int iters, int in_flight, int blocks,
                          const void* buf, float* out, uint64_t* clocks, hipStream_t s) {
  const uint32_t records = uint32_t((int64_t(16) << 20) + int64_t(blocks) * cold_bytes);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  if (in_flight == 1)
    k_delivery_probe<1><<<blocks, 512, 0, s>>>(b, records, uint32_t(cold_bytes), hot_pct, iters, out, clocks);
  else
    k_delivery_probe<2><<<blocks, 512, 0, s>>>(b, records, uint32_t(cold_bytes), hot_pct, iters, out, clocks);
  return check_launch("delivery probe");
}

int launch_mfma_ceiling(int shape, int iters, int blocks, float* out, hipStream_t s) {
  if (shape == 0) k_mfma_ceiling<0><<<blocks, 512, 0, s>>>(out, iters, 1e-3f);
  else if (shape == 1) k_mfma_ceiling<1><<<blocks, 512, 0, s>>>(out, iters, 1e-3f);
  else k_mfma_ceiling<2><<<blocks, 512, 0, s>>>(out, iters, 1e-3f);
  return check_launch("mfma ceiling");
}

}  // namespace fsm
