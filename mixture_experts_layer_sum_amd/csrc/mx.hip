// MXFP8 expert products for gfx950.
//
// FarSkip-Collective's inference runs use FP8 quantisation with fused MoE forward kernels (the
// page's experimental setup, inference parameters); the format taken is OCP MXFP8, which CDNA4's
// scaled matrix instruction executes natively: E4M3 elements, one E8M0 power-of-two scale per 32
// consecutive elements along the reduction dimension K.  Block scale: the smallest 2^s with
// max|x| / 2^s <= 448 (nothing saturates); elements x / 2^s rounded to the nearest E4M3 value,
// ties to the even code.
//
//   k_mx_quantize  bf16 rows -> E4M3 codes + E8M0 scales (activations each call, weights once)
//   k_gemm_mx      the expert MLP of section 2.1 on MXFP8 operands, as two grouped products:
//                    gate/up: H = (X W1^T) . SiLU(X W2^T), formed in fp32 from the dequantised
//                             accumulators and quantised to MXFP8 in the epilogue (one wave's 32
//                             H columns of a row are exactly one block)
//                    down:    Y = H W3^T in bf16
//
// v_mfma_scale_f32_16x16x128_f8f6f4 operand layout (measured on the device): lane l holds row
// l % 16 of its operand and 32 K values, K = 16 (l / 16) .. +15 in bytes 0-15 and
// K = 64 + 16 (l / 16) .. +15 in bytes 16-31; the scale byte in lane l is the scale of K block
// l / 16 (K 32 (l / 16) .. +31) of row l % 16.  The product is C[4 (l / 16) + r][l % 16] of
// (first operand) x (second operand)^T in accumulator element r, as for the bf16 instruction, so
// passing the weight fragment first again leaves four consecutive output columns in a lane.
//
// A stage holds 128 K values per row (128 bytes, the same LDS row geometry as the bf16 kernel's
// 64 bf16 values) for BM + BN rows, loaded straight into LDS, plus their 4 scale bytes per row.
// Rows' scales lie K / 32 bytes apart, so a load of one row's 4 bytes per lane touches a cache line
// per row; with two stages and K a multiple of 512, the 256-row tiles load each row's scales for
// four stages at once (16 bytes per lane, a quarter of the cache-line lookups), into a
// double-buffered block beside the stage ring: gate/up 15.4 -> 13.6 ms and down 8.4 -> 8.0 ms on
// the DeepSeek-V3 layer, bit for bit the same output.
#include "common.h"
#include "tile_kit.h"

namespace fsm {

typedef int mx_v8i __attribute__((ext_vector_type(8)));

// ---- numbers -------------------------------------------------------------------------------
// Shared exponent of a block whose largest magnitude is amax: the smallest s with
// amax <= 448 * 2^s (448 = 0.875 * 2^9), 0 for an all-zero block, clamped to the E8M0 range.
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  const float f = frexpf(amax, &e);   // amax = f * 2^e, f in [0.5, 1), exact
  const int s = e - 9 + (f > 0.875f ? 1 : 0);
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// Four E4M3 codes of a, b, c, d divided by 2^s, packed little-endian into one word. gfx950's scaled
// pair conversion divides by its scale operand and rounds to the nearest code, ties to even, keeping
// the sign of zero; for every value whose quotient lies within +-448 (which the block exponent makes
// true of a whole block) that is the format's round-to-nearest-even encoding, subnormals included.
typedef short mx_v2i16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3_word(float a, float b, float c, float d, int s) {
  const float scale = ldexpf(1.0f, s);   // 2^s; 2^-127 is an fp32 subnormal and still exact
  mx_v2i16 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, scale, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, scale, true);
  return uint32_t(uint16_t(w[0])) | (uint32_t(uint16_t(w[1])) << 16);
}

// ---- quantize ------------------------------------------------------------------------------
// One thread per 32-element block of a row: 64 bytes of bf16 in, 32 code bytes and one scale out.
__global__ __launch_bounds__(256) void k_mx_quantize(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = K / 32;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * nb) return;
  const int64_t row = i / nb, blk = i - row * nb;
  const uint4* src = reinterpret_cast<const uint4*>(X + row * K + blk * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) unpack8(src[q], v + 8 * q);
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
  const int s = mx_block_exp(amax);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    w[q] = e4m3_word(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], s);
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + row * K + blk * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[row * nb + blk] = uint8_t(s + 127);
}

// ---- grouped product -----------------------------------------------------------------------
enum { MX_PLAIN = 0, MX_SWIGLU = 1 };
// MX_ROWS_SINGLE reads rows as MX_ROWS_GROUPED does; a single-group call (the shared expert) uses it
// so that profilers report it apart from the routed products
enum { MX_ROWS_GROUPED = 0, MX_ROWS_SINGLE = 1, MX_ROWS_GATHER = 2 };

struct MxArgs {
  const uint8_t* A;          // [rows, K] E4M3 codes
  const uint8_t* As;         // [rows, K / 32] E8M0 scales
  const uint8_t* B1;         // [G, n_b, K] (n_b = n_out, or c for SwiGLU)
  const uint8_t* B1s;        // [G, n_b, K / 32]
  const uint8_t* B2;         // SwiGLU gate weights, same layout
  const uint8_t* B2s;
  void* out;                 // MX_PLAIN: bf16 [rows, n_out]; MX_SWIGLU: codes [rows, n_out]
  uint8_t* out_s;            // MX_SWIGLU: scales [rows, n_out / 32]
  const int32_t* offsets;
  const int32_t* tile_start;
  const int32_t* tile_group;
  int64_t b_group_stride;    // bytes between groups of B1 / B2 codes (n_b * K)
  int64_t bs_group_stride;   // bytes between groups of B1s / B2s (n_b * K / 32)
  int32_t K, n_out, M, G, n_tiles, group_m, quad_nb;
  const int32_t* gather;     // MX_ROWS_GATHER: grouped row r reads A row gather[r] / gather_k
  int32_t gather_k;
  int64_t a_rows;            // rows of A (the gathered form's resource extent)
};

// Tilings: BM x 256 output tiles, WAVES_M x 4 waves, S LDS stages.  256 x 256 with 8 waves and two
// stages for the prefill-sized groups; 64 x 256 with 4 waves and three stages for groups of a few
// dozen rows (a decode batch), where the product streams the weights and more bytes in flight per
// CU matter more than the MFMA work.  Both sum every output over K in the same order.
// BNT: the weight codes are loaded with the nontemporal hint (groups that fit in one M-tile, whose
// weight lines no other workgroup reads).
template <int EPI, int ROWS, int BM_ = 256, int WAVES_M_ = 2, int S_ = 2, bool SB = false, bool BNT = false>
__global__ __launch_bounds__(256 * WAVES_M_) void k_gemm_mx(MxArgs p) {
  constexpr int BM = BM_, BN = 256, WAVES_M = WAVES_M_, WAVES_N = 4, NW = WAVES_M * WAVES_N, S = S_;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 16, FN = WTN / 16;
  constexpr int RB = 128;                       // bytes (K values) per LDS row per stage
  constexpr int RUN_ROWS = 8;                   // rows of one wave's 1 KB direct-to-LDS run
  constexpr int A_RUNS = BM / RUN_ROWS / NW, B_RUNS = BN / RUN_ROWS / NW;
  // scale bytes: the BM + BN rows' 4 bytes per stage, in runs of 64 rows (one 4-byte load per
  // lane); wave w loads runs w, w + NW, ...  Runs past the last row load zeros into padding, so
  // every wave issues the same number of loads per stage.
  constexpr int SROWS = BM + BN, SL = (SROWS + 64 * NW - 1) / (64 * NW);
  constexpr int LOADS = A_RUNS + B_RUNS + SL;   // vector-memory operations per wave per stage
  constexpr int DATA = (BM + BN) * RB, SCL = SL * NW * 64 * 4;
  // SB: the scale bytes of four stages at a time (each row's 16 bytes, one 16-byte load per lane,
  // so a run of 64 rows touches 64 cache lines once per four stages instead of once per stage),
  // double-buffered; the block of stages 4m .. 4m + 3 is requested with stage 4m's data
  static_assert(!SB || S == 2, "scale blocks with two stages");
  constexpr int SBLK = SL * NW * 64 * 16;
  static_assert(EPI != MX_SWIGLU || (FN % 2) == 0, "SwiGLU needs paired fragments");
  static_assert(EPI != MX_SWIGLU || (WTN / 2) == 32, "a wave's H columns of a row must be one MX block");
  static_assert(A_RUNS * RUN_ROWS * NW == BM && B_RUNS * RUN_ROWS * NW == BN, "runs must tile the stage");
  static_assert(BM % 64 == 0 && (BN / 2) % 64 == 0, "scale runs must not straddle A / B / gate rows");
  static_assert(S == 2 || S == 3, "two or three stages");
  static_assert(LOADS * (S - 2) < 64, "vmcnt range");

  // one LDS array per stage (data rows, then their scale bytes): separate objects let the compiler
  // see that the loads filling one stage never alias the reads of the other
  constexpr int STAGE = DATA + (SB ? 0 : SCL);
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE], st1[STAGE], st2[S > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sbk[SB ? 2 * SBLK : 16];
#define MX_SM(BUF) ((BUF) == 0 ? st0 : (BUF) == 1 ? st1 : st2)

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int mt, nt;
  if (!map_tile(p, BM, mt, nt)) return;
  int g, row0, rows;
  if (!resolve_mtile(p, mt, BM, g, row0, rows)) return;

  const int K = p.K, KB = K / 32;               // scale bytes per row
  const int n0 = EPI == MX_SWIGLU ? nt * (BN / 2) : nt * BN;
  const int nvalid = min(EPI == MX_SWIGLU ? BN / 2 : BN, p.n_out - n0);
  // data resources: rows past `rows` (A) or `nvalid` (B) lie beyond them and load as zeros
  const __amdgpu_buffer_rsrc_t rA =
      ROWS == MX_ROWS_GATHER ? make_rsrc(p.A, p.a_rows * K) : make_rsrc(p.A + int64_t(row0) * K, int64_t(rows) * K);
  const __amdgpu_buffer_rsrc_t rAs =
      ROWS == MX_ROWS_GATHER ? make_rsrc(p.As, p.a_rows * KB) : make_rsrc(p.As + int64_t(row0) * KB, int64_t(rows) * KB);
  const int wb_row0 = wave * B_RUNS * RUN_ROWS;   // first B tile row of this wave's data runs
  const bool b_gate = EPI == MX_SWIGLU && wb_row0 >= BN / 2;
  const __amdgpu_buffer_rsrc_t rB = make_rsrc((b_gate ? p.B2 : p.B1) + g * p.b_group_stride + int64_t(n0) * K,
                                              int64_t(nvalid) * K);
  // scale rows: run i of this wave covers tile rows 64 (i NW + wave) + lane (A rows first, then B
  // rows); a run lies wholly in A, in B1's half or in B2's half (uniform over the wave)
  const __amdgpu_buffer_rsrc_t rB1s = make_rsrc(p.B1s + g * p.bs_group_stride + int64_t(n0) * KB, int64_t(nvalid) * KB);
  const __amdgpu_buffer_rsrc_t rB2s =
      EPI == MX_SWIGLU ? make_rsrc(p.B2s + g * p.bs_group_stride + int64_t(n0) * KB, int64_t(nvalid) * KB) : rB1s;

  // this lane's load offsets at k = 0 (lane l writes physical chunk l % 8 of row l / 8 of a run,
  // so it loads logical chunk (l % 8) ^ (row & 7): the XOR swizzle the fragment reads undo)
  const int d_row = lane >> 3, d_ch = (lane & 7) ^ d_row;
  uint32_t dA[A_RUNS], dB[B_RUNS], dS[SL];
  __amdgpu_buffer_rsrc_t rS[SL];
  if (ROWS == MX_ROWS_GATHER) {
    int src[A_RUNS];
#pragma unroll
    for (int i = 0; i < A_RUNS; ++i)
      src[i] = p.gather[row0 + min((wave * A_RUNS + i) * RUN_ROWS + d_row, rows - 1)] / p.gather_k;
#pragma unroll
    for (int i = 0; i < A_RUNS; ++i) {
      const int r = (wave * A_RUNS + i) * RUN_ROWS + d_row;
      dA[i] = r < rows ? uint32_t(src[i]) * uint32_t(K) + uint32_t(d_ch) * 16u : 0x80000000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < A_RUNS; ++i) dA[i] = uint32_t((wave * A_RUNS + i) * RUN_ROWS + d_row) * uint32_t(K) + uint32_t(d_ch) * 16u;
  }
#pragma unroll
  for (int i = 0; i < B_RUNS; ++i) {
    const int r = wb_row0 + i * RUN_ROWS + d_row;
    dB[i] = uint32_t(b_gate ? r - BN / 2 : r) * uint32_t(K) + uint32_t(d_ch) * 16u;
  }
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const int s_row0 = (i * NW + wave) * 64, s_row = s_row0 + lane;   // s_row0 is wave-uniform
    if (s_row0 >= SROWS) {          // padding run: beyond every resource, loads zeros
      rS[i] = rAs;
      dS[i] = 0x80000000u;
    } else if (s_row0 < BM) {       // A rows
      rS[i] = rAs;
      if (ROWS == MX_ROWS_GATHER)
        dS[i] = s_row < rows ? uint32_t(p.gather[row0 + s_row] / p.gather_k) * uint32_t(KB) : 0x80000000u;
      else
        dS[i] = uint32_t(s_row) * uint32_t(KB);
    } else {                        // B rows (the gate half reads B2's scales)
      const int b_row = s_row - BM;
      const bool s_gate = EPI == MX_SWIGLU && s_row0 - BM >= BN / 2;
      rS[i] = s_gate ? rB2s : rB1s;
      dS[i] = uint32_t(s_gate ? b_row - BN / 2 : b_row) * uint32_t(KB);
    }
  }

  // fragment reads: A rows (wm * WTM + 16 i + lane % 16), B rows likewise; lane group q = lane / 16
  // takes the 16-byte chunks q and q + 4 of its row (K 16q .. and 64 + 16q ..), swizzled by row & 7,
  // and the scale byte of K block q.  Per-lane bases; the row-block terms are constants that fold
  // into the reads' immediate offsets.
  const int q = lane >> 4, sw = lane & 7;
  const int ch_lo = (q ^ sw) << 4, ch_hi = ((q + 4) ^ sw) << 4;
  const int fa0 = wm * WTM + (lane & 15);
  const int fb0 = BM + (EPI == MX_SWIGLU ? wn * (WTN / 2) : wn * WTN) + (lane & 15);
  const int a_lo = fa0 * RB + ch_lo, a_hi = fa0 * RB + ch_hi, a_sc = DATA + fa0 * 4 + q;
  const int b_lo = fb0 * RB + ch_lo, b_hi = fb0 * RB + ch_hi, b_sc = DATA + fb0 * 4 + q;
  const int a_scb = fa0 * 16 + q, b_scb = fb0 * 16 + q;   // SB: scale row offsets within a block

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t kb_zero;   // opaque zero: every load's voffset is a fresh register (see the bf16 kernel)
  asm volatile("s_mov_b32 %0, 0" : "=s"(kb_zero));
#define MX_STAGE(KT, BUF)                                                                       \
  {                                                                                             \
    const uint32_t kb = uint32_t(KT) * RB + kb_zero;                                            \
    _Pragma("unroll") for (int i = 0; i < A_RUNS; ++i)                                          \
      FSM_LDS_DMA16(rA, &MX_SM(BUF)[(wave * A_RUNS + i) * RUN_ROWS * RB], dA[i] + kb); \
    _Pragma("unroll") for (int i = 0; i < B_RUNS; ++i) {                                        \
      if (BNT) FSM_LDS_DMA16_NT(rB, &MX_SM(BUF)[(BM + wb_row0 + i * RUN_ROWS) * RB], dB[i] + kb); \
      else FSM_LDS_DMA16(rB, &MX_SM(BUF)[(BM + wb_row0 + i * RUN_ROWS) * RB], dB[i] + kb);      \
    }                                                                                           \
    if (!SB) {                                                                                  \
      _Pragma("unroll") for (int i = 0; i < SL; ++i)                                            \
        FSM_LDS_DMA4(rS[i], &MX_SM(BUF)[DATA + (i * NW + wave) * 64 * 4], dS[i] + uint32_t(KT) * 4u + kb_zero); \
    } else if (((KT) & 3) == 0) {                                                               \
      const uint32_t m_ = uint32_t(KT) >> 2;                                                    \
      _Pragma("unroll") for (int i = 0; i < SL; ++i)                                            \
        FSM_LDS_DMA16(rS[i], &sbk[(m_ & 1u) * SBLK + (i * NW + wave) * 64 * 16], dS[i] + m_ * 16u + kb_zero); \
    }                                                                                           \
  }
#define MX_BROW(J) \
  ((EPI == MX_SWIGLU) ? ((J) < FN / 2 ? (J) * 16 : BN / 2 + ((J) - FN / 2) * 16) : (J) * 16)
#define MX_LD16(BUF, OFF) (*reinterpret_cast<const uint4*>(&MX_SM(BUF)[(OFF)]))
#define MX_FRAG(BUF, LO, HI, OUT)                                                               \
  {                                                                                             \
    const uint4 lo_ = MX_LD16(BUF, LO), hi_ = MX_LD16(BUF, HI);                                 \
    OUT = mx_v8i{int(lo_.x), int(lo_.y), int(lo_.z), int(lo_.w), int(hi_.x), int(hi_.y), int(hi_.z), int(hi_.w)}; \
  }
#define MX_FRAG_A(BUF, I, OUT) MX_FRAG(BUF, a_lo + (I) * 16 * RB, a_hi + (I) * 16 * RB, OUT)
#define MX_FRAG_B(BUF, J, OUT) MX_FRAG(BUF, b_lo + MX_BROW(J) * RB, b_hi + MX_BROW(J) * RB, OUT)
#define MX_SC_A(BUF, I) (SB ? int(sbk[sc_off + a_scb + (I) * 256]) : int(MX_SM(BUF)[a_sc + (I) * 64]))
#define MX_SC_B(BUF, J) (SB ? int(sbk[sc_off + b_scb + MX_BROW(J) * 16]) : int(MX_SM(BUF)[b_sc + MX_BROW(J) * 4]))
  // one stage: the first A fragment, then the B fragments (so the first MFMA waits only for the
  // first A and B fragment), then per A row block the next block's fragment and scale are read
  // before the current block's FN MFMAs; scheduling groups pin that order so an LDS read is always
  // in flight under FN MFMAs
#define MX_COMPUTE(BUF)                                                                         \
  {                                                                                             \
    mx_v8i bf[FN], a_cur, a_nxt;                                                                \
    int bsc[FN], as_cur, as_nxt;                                                                \
    MX_FRAG_A(BUF, 0, a_cur);                                                                   \
    as_cur = MX_SC_A(BUF, 0);                                                                   \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                            \
      __builtin_amdgcn_sched_barrier(0);                                                        \
      MX_FRAG_B(BUF, j, bf[j]);                                                                 \
      bsc[j] = MX_SC_B(BUF, j);                                                                 \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                            \
      if (i + 1 < FM) {                                                                         \
        MX_FRAG_A(BUF, i + 1, a_nxt);                                                           \
        as_nxt = MX_SC_A(BUF, i + 1);                                                           \
      }                                                                                         \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                            \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], a_cur, acc[i][j], 0, 0, 0, \
                                                                     bsc[j], 0, as_cur);        \
      if (i + 1 < FM) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                        \
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                       \
      a_cur = a_nxt;                                                                            \
      as_cur = as_nxt;                                                                          \
    }                                                                                           \
  }
#define MX_BARRIER()                    \
  {                                     \
    asm volatile("" ::: "memory");      \
    __builtin_amdgcn_s_barrier();       \
    asm volatile("" ::: "memory");      \
  }

  const int KT = K / RB;
  // A wave whose rows all lie past the group's last row (the ragged last M-tile of a group; most of
  // the tile for a decode batch of a few dozen rows per expert) skips its fragment reads and MFMAs.
  // It still loads its share of every stage and meets every barrier; its rows are never stored.
  const bool live = wm * WTM < rows;
  // ring of S stages: stages 0 .. S-2 in flight, then wait for stage 0 (straight-line branches, so
  // the compiler's own wait-count tracking sees which stages are pending)
  if (KT >= S - 1) {
#pragma unroll
    for (int st = 0; st < S - 1; ++st) MX_STAGE(st, st);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS * (S - 2)));
  } else {
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < KT) MX_STAGE(st, st);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  MX_BARRIER();
  // one ring step on buffer J: refill the buffer read one step earlier with stage kt + S - 1, run
  // this stage's MFMAs, then wait until the next stage is in LDS for every wave
#define MX_RING_STEP(J)                                                                         \
  {                                                                                             \
    if (kt + S - 1 < KT) MX_STAGE(kt + S - 1, ((J) + S - 1) % S);                               \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    const int sc_off = SB ? ((kt >> 2) & 1) * SBLK + (kt & 3) * 4 : 0;                          \
    (void)sc_off;                                                                               \
    if (live) MX_COMPUTE(J)                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    if (++kt >= KT) break;                                                                      \
    if (kt + S - 2 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS * (S - 2)));               \
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                                             \
    MX_BARRIER();                                                                               \
  }
  for (int kt = 0;;) {   // unrolled S times so each step names its buffers as constants
    MX_RING_STEP(0);
    MX_RING_STEP(1);
    if (S > 2) MX_RING_STEP(2 % S);
  }
#undef MX_RING_STEP
  (void)LOADS;
#undef MX_SM
#undef MX_STAGE
#undef MX_BROW
#undef MX_LD16
#undef MX_FRAG
#undef MX_FRAG_A
#undef MX_FRAG_B
#undef MX_SC_A
#undef MX_SC_B
#undef MX_COMPUTE
#undef MX_BARRIER

  // epilogue: lane holds rows m = .. + (lane & 15), columns n = .. + 4 (lane >> 4) + {0..3}
  const int ml = lane & 15, nl = q * 4;
  if (EPI == MX_PLAIN && FN % 2 == 0 && (nt + 1) * BN <= p.n_out) {
    // adjacent fragments paired into 16-byte stores (pair_words); partner lanes share their row
    const int pc = pair_col(lane);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = wm * WTM + i * 16 + ml;
      if (m >= rows) continue;
      uint16_t* out = static_cast<uint16_t*>(p.out) + int64_t(row0 + m) * p.n_out + nt * BN + wn * WTN + pc;
#pragma unroll
      for (int j = 0; j + 1 < FN; j += 2) {
        const f32x4 a = acc[i][j], b = acc[i][j + 1];
        *reinterpret_cast<st_u32x4*>(out + j * 16) =
            pair_words(pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]), pack2(b[2], b[3]));
      }
    }
  } else if (EPI == MX_PLAIN) {
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = wm * WTM + i * 16 + ml;
      if (m >= rows) continue;
      const int64_t orow = int64_t(row0 + m);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = nt * BN + wn * WTN + j * 16 + nl;
        if (col >= p.n_out) continue;
        const f32x4 a = acc[i][j];
        uint2 v;
        v.x = pack2(a[0], a[1]);
        v.y = pack2(a[2], a[3]);
        *reinterpret_cast<uint2*>(out + orow * p.n_out + col) = v;
      }
    }
  } else {
    // H = U . SiLU(G) in fp32 (the reciprocal to within one ulp), then MXFP8: a wave's 32 H columns of one row are one block, held by
    // the four lanes with the same lane % 16 (8 values each); the block maximum is a two-step
    // cross-lane max.
    uint8_t* hq = static_cast<uint8_t*>(p.out);
    const int hcol0 = nt * (BN / 2) + wn * (WTN / 2);   // first H column of this wave (block aligned)
    const int nb = p.n_out / 32;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float h[FN / 2][4];
      float amax = 0.f;
#pragma unroll
      for (int jj = 0; jj < FN / 2; ++jj) {
        const f32x4 u = acc[i][jj], gt = acc[i][jj + FN / 2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          h[jj][r] = u[r] * gt[r] * __builtin_amdgcn_rcpf(1.0f + __expf(-gt[r]));
          amax = fmaxf(amax, fabsf(h[jj][r]));
        }
      }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const int s = mx_block_exp(amax);
      const int m = wm * WTM + i * 16 + ml;
      if (m >= rows || hcol0 >= p.n_out) continue;
      const int64_t orow = int64_t(row0 + m);
#pragma unroll
      for (int jj = 0; jj < FN / 2; ++jj) {
        const uint32_t w = e4m3_word(h[jj][0], h[jj][1], h[jj][2], h[jj][3], s);
        *reinterpret_cast<uint32_t*>(hq + orow * p.n_out + hcol0 + jj * 16 + nl) = w;
      }
      if (q == 0) p.out_s[orow * nb + hcol0 / 32] = uint8_t(s + 127);
    }
  }
}

// ---- host launchers ------------------------------------------------------------------------
namespace {
constexpr int MX_BM = 256, MX_BN = 256, MX_GROUP_M = 4, MX_SMALL_BM = 64, MX_SMALL_ROWS = 96;

// 64-row tiles where groups average at most MX_SMALL_ROWS rows, or where 256-row tiles would not
// give every CU a workgroup (the rule of the bf16 product)
bool mx_small(int64_t N, int32_t G, int64_t c) {
  return N <= int64_t(MX_SMALL_ROWS) * G || (cdiv(N, MX_BM) + G) * cdiv(c, MX_BN / 2) < 256;
}
int mx_bm(int64_t N, int32_t G, int64_t c) { return mx_small(N, G, c) ? MX_SMALL_BM : MX_BM; }
// routed groups that average at most one 64-row tile stream their weights (read once) past the caches
bool mx_stream_b(int64_t N, int32_t G) { return G > 1 && N <= int64_t(MX_SMALL_BM) * G; }
int64_t mx_max_tiles(int64_t N, int32_t G, int bm) { return cdiv(N, bm) + G; }

// workspace: the M-tile table, then (fused call only) H's codes and scales
struct MxWs {
  int32_t* ts;
  int32_t* grp;
  uint8_t* Hq;
  uint8_t* Hs;
};

MxWs carve_mx(void* ws, int32_t G, int64_t N, int64_t c, size_t* total) {
  size_t off = 0;
  MxWs w;
  char* base = static_cast<char*>(ws);
  w.ts = reinterpret_cast<int32_t*>(base + off);
  off = align_up(off + size_t(G + 1) * 4, 256);
  w.grp = reinterpret_cast<int32_t*>(base + off);
  off = align_up(off + size_t(mx_max_tiles(N, G, MX_SMALL_BM)) * 4, 256);   // room for either tiling
  w.Hq = reinterpret_cast<uint8_t*>(base + off);
  off = align_up(off + size_t(N) * size_t(c), 256);
  w.Hs = reinterpret_cast<uint8_t*>(base + off);
  off = align_up(off + size_t(N) * size_t(c / 32), 256);
  if (total) *total = off;
  return w;
}

int mx_gate_up(const uint8_t* Xq, const uint8_t* Xs, const int32_t* offsets, int32_t G, const uint8_t* W1q,
               const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s, int64_t N, int64_t d, int64_t c,
               uint8_t* Hq, uint8_t* Hs, const MxWs& w, hipStream_t s, const int32_t* gather, int32_t gather_k,
               int64_t x_rows, int bm) {
  MxArgs a{};
  a.A = Xq; a.As = Xs; a.B1 = W1q; a.B1s = W1s; a.B2 = W2q; a.B2s = W2s;
  a.out = Hq; a.out_s = Hs;
  a.offsets = offsets; a.tile_start = w.ts; a.tile_group = w.grp;
  a.b_group_stride = c * d; a.bs_group_stride = c * (d / 32);
  a.K = int32_t(d); a.n_out = int32_t(c); a.M = int32_t(N); a.G = G; a.group_m = MX_GROUP_M;
  a.n_tiles = int32_t(cdiv(c, MX_BN / 2));
  a.quad_nb = quad_width(a.n_tiles, a.group_m);
  a.gather = gather; a.gather_k = gather_k; a.a_rows = x_rows;
  ProfScope prof(G > 1 ? MOE_K_MX_GATE_UP : MOE_K_MX_DENSE_GATE_UP, s);
  const dim3 grid(unsigned(quad_grid(mx_max_tiles(N, G, bm), a.n_tiles, a.group_m, a.quad_nb)));
  const bool stream_b = mx_stream_b(N, G);
  if (bm == MX_SMALL_BM && gather && stream_b)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GATHER, MX_SMALL_BM, 1, 3, false, true><<<grid, 256, 0, s>>>(a);
  else if (bm == MX_SMALL_BM && gather)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GATHER, MX_SMALL_BM, 1, 3><<<grid, 256, 0, s>>>(a);
  else if (bm == MX_SMALL_BM && G == 1)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_SINGLE, MX_SMALL_BM, 1, 3><<<grid, 256, 0, s>>>(a);
  else if (bm == MX_SMALL_BM && stream_b)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GROUPED, MX_SMALL_BM, 1, 3, false, true><<<grid, 256, 0, s>>>(a);
  else if (bm == MX_SMALL_BM)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GROUPED, MX_SMALL_BM, 1, 3><<<grid, 256, 0, s>>>(a);
  else if (d % 512 == 0 && gather)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GATHER, 256, 2, 2, true><<<grid, 512, 0, s>>>(a);
  else if (d % 512 == 0 && G == 1)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_SINGLE, 256, 2, 2, true><<<grid, 512, 0, s>>>(a);
  else if (d % 512 == 0)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GROUPED, 256, 2, 2, true><<<grid, 512, 0, s>>>(a);
  else if (gather)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GATHER><<<grid, 512, 0, s>>>(a);
  else if (G == 1)
    k_gemm_mx<MX_SWIGLU, MX_ROWS_SINGLE><<<grid, 512, 0, s>>>(a);
  else
    k_gemm_mx<MX_SWIGLU, MX_ROWS_GROUPED><<<grid, 512, 0, s>>>(a);
  return check_launch("mx grouped gemm phase 1");
}

int mx_down(const uint8_t* Hq, const uint8_t* Hs, const int32_t* offsets, int32_t G, const uint8_t* W3q,
            const uint8_t* W3s, int64_t N, int64_t c, int64_t d, void* Y, const MxWs& w, hipStream_t s, int bm) {
  MxArgs a{};
  a.A = Hq; a.As = Hs; a.B1 = W3q; a.B1s = W3s; a.B2 = nullptr; a.B2s = nullptr;
  a.out = Y; a.out_s = nullptr;
  a.offsets = offsets; a.tile_start = w.ts; a.tile_group = w.grp;
  a.b_group_stride = d * c; a.bs_group_stride = d * (c / 32);
  a.K = int32_t(c); a.n_out = int32_t(d); a.M = int32_t(N); a.G = G; a.group_m = MX_GROUP_M;
  a.n_tiles = int32_t(cdiv(d, MX_BN));
  a.quad_nb = quad_width(a.n_tiles, a.group_m);
  ProfScope prof(G > 1 ? MOE_K_MX_DOWN : MOE_K_MX_DENSE_DOWN, s);
  const dim3 grid(unsigned(quad_grid(mx_max_tiles(N, G, bm), a.n_tiles, a.group_m, a.quad_nb)));
  if (bm == MX_SMALL_BM && G == 1)
    k_gemm_mx<MX_PLAIN, MX_ROWS_SINGLE, MX_SMALL_BM, 1, 3><<<grid, 256, 0, s>>>(a);
  else if (bm == MX_SMALL_BM && mx_stream_b(N, G))
    k_gemm_mx<MX_PLAIN, MX_ROWS_GROUPED, MX_SMALL_BM, 1, 3, false, true><<<grid, 256, 0, s>>>(a);
  else if (bm == MX_SMALL_BM)
    k_gemm_mx<MX_PLAIN, MX_ROWS_GROUPED, MX_SMALL_BM, 1, 3><<<grid, 256, 0, s>>>(a);
  else if (c % 512 == 0 && G == 1)
    k_gemm_mx<MX_PLAIN, MX_ROWS_SINGLE, 256, 2, 2, true><<<grid, 512, 0, s>>>(a);
  else if (c % 512 == 0)
    k_gemm_mx<MX_PLAIN, MX_ROWS_GROUPED, 256, 2, 2, true><<<grid, 512, 0, s>>>(a);
  else if (G == 1)
    k_gemm_mx<MX_PLAIN, MX_ROWS_SINGLE><<<grid, 512, 0, s>>>(a);
  else
    k_gemm_mx<MX_PLAIN, MX_ROWS_GROUPED><<<grid, 512, 0, s>>>(a);
  return check_launch("mx grouped gemm phase 2");
}
}  // namespace

int launch_mx_quantize(const void* X, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t blocks = rows * (K / 32);
  if (blocks == 0) return MOE_OK;
  ProfScope prof(MOE_K_MX_QUANTIZE, s);
  k_mx_quantize<<<unsigned(cdiv(blocks, 256)), 256, 0, s>>>(static_cast<const uint16_t*>(X), rows, K, codes, scales);
  return check_launch("mx quantize");
}

size_t mx_swiglu_ws_bytes(int64_t N, int32_t G, int64_t c) {
  size_t total = 0;
  carve_mx(nullptr, G, N, c, &total);
  return total;
}

int launch_grouped_swiglu_mx(const uint8_t* Xq, const uint8_t* Xs, const int32_t* offsets, int32_t G,
                             const uint8_t* W1q, const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s,
                             const uint8_t* W3q, const uint8_t* W3s, int64_t N, int64_t d, int64_t c, void* Y,
                             void* ws, hipStream_t s, const int32_t* gather, int32_t gather_k, int64_t x_rows,
                             int phases, uint8_t* Hq, uint8_t* Hs, hipEvent_t mid) {
  // phases: 3 = both (H in the workspace), 1 = gate/up into the caller's Hq / Hs, 2 = down from them
  MxWs w = carve_mx(ws, G, N, phases == 3 ? c : 0, nullptr);
  if (N == 0) {   // nothing to compute; the phase event still marks this point of the stream
    const hipError_t e = mid ? hipEventRecord(mid, s) : hipSuccess;
    return e == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  if (phases == 3) {
    Hq = w.Hq;
    Hs = w.Hs;
  }
  // the tiling follows the group sizes and the hidden width, so the two calls of a split product
  // (phases 1 then 2) pick the same one
  const int bm = mx_bm(N, G, c);
  if (int rc = launch_tile_table(offsets, G, bm, int(mx_max_tiles(N, G, bm)), w.ts, w.grp, s)) return rc;
  if (phases & 1)
    if (int rc = mx_gate_up(Xq, Xs, offsets, G, W1q, W1s, W2q, W2s, N, d, c, Hq, Hs, w, s, gather, gather_k, x_rows,
                            bm))
      return rc;
  if (mid) {
    const hipError_t e = hipEventRecord(mid, s);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  if (phases & 2) return mx_down(Hq, Hs, offsets, G, W3q, W3s, N, c, d, Y, w, s, bm);
  return MOE_OK;
}

}  // namespace fsm
