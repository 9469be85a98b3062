// Grouped SwiGLU GEMM pair and the router GEMM for gfx950.
//
// The expert MLP of "FarSkip-Collective" section 2.1, MLP(A) = sigma(A W1^T . g(A W2^T)) W3^T with
// g = SiLU and sigma = identity, is run as two contractions per expert group:
//   phase 1:  H = (X W1^T) . SiLU(X W2^T)    one tile holds matching columns of W1 and W2, so the
//                                             SwiGLU product is formed in registers (no U/G in HBM)
//   phase 2:  Y = H W3^T
// Both are "NT" products (both operands contiguous along K), which is the layout the bf16 MFMA
// wants.  The router logits A W_R^T (section 2.1, G(A) = s(A W_R^T)) use the same tile kernel with
// a float32 epilogue.
//
// Tile kernel: BM x BN output tile per workgroup, BK = 64, waves laid out WAVES_M x WAVES_N, each
// wave owning a (BM/WAVES_M) x (BN/WAVES_N) block of v_mfma_f32_16x16x32_bf16 tiles.  Global
// tiles go straight from HBM into a ring of LDS stages with direct-to-LDS buffer loads (no
// register staging, one barrier per K step); LDS rows are 128 bytes and their eight 16-byte
// chunks are XOR-swizzled with the row index so that the MFMA fragment reads (16 rows x one
// chunk per 16 lanes) are bank-conflict free.  The MFMA is issued
// with the weight fragment as its first operand, which leaves every lane holding four consecutive
// output columns of one row: the epilogue stores 8-byte (bf16) or 16-byte (fp32) vectors.
//
// Groups (experts) have data-dependent row counts that stay on the device: a one-block kernel
// turns the group offsets into a prefix sum of M-tiles per group and a map from M-tile to group,
// which each workgroup reads with one scalar load.  The grid is sized for the worst case
// (ceil(N/BM) + G M-tiles); the surplus workgroups exit at once.
#include "common.h"
#include "tile_kit.h"

namespace fsm {

// EPI_UG: the SwiGLU tile's loads (W1 and W2 columns side by side), storing U and G themselves
// into [rows, 2 n_out] (U in columns [0, n_out), G in [n_out, 2 n_out)) for a backward pass.
enum { EPI_PLAIN = 0, EPI_SWIGLU = 1, EPI_F32_BIAS = 2, EPI_UG = 3 };

struct GemmArgs {
  const void* A;              // [rows, K]
  const void* B1;             // [G, n_b, K] (n_b = n_out, or c for SwiGLU)
  const void* B2;             // SwiGLU gate weights, same layout as B1
  void* out;                  // [rows, n_out]
  const float* bias;          // EPI_F32_BIAS: [n_out] or null
  const int32_t* offsets;     // [G+1] or null (dense: rows [0, M))
  const int32_t* tile_start;  // [G+1] M-tile prefix per group, or null
  const int32_t* tile_group;  // [max M-tiles] group of each M-tile (-1 = surplus), or null
  int64_t b_group_stride;     // elements between consecutive groups of B1/B2
  int32_t K, n_out, M, G, n_tiles;
  int32_t group_m;            // M-tiles per scheduling group (tiles of a group share weights)
  const int32_t* gather;      // ROWS_GATHER: grouped row r reads A row gather[r] / gather_k
  int32_t gather_k;
  int64_t a_rows;             // ROWS_GATHER: rows of A (its buffer-resource extent)
  int32_t quad_nb;            // > 0: the 2 x 2 XCD-block order below, with quad_nb N-tiles per block
  // K-major B (the backward's row modes): B1, B2 are [K rows, ldb] per group, as the weights are
  // stored; rows [0, b_k1) of B1 hold data (later rows read as zeros), and with b_ksplit > 0,
  // rows k >= b_ksplit are row k - b_ksplit of B2
  int64_t ldb, b_k1;
  int32_t b_ksplit;
};

// How a workgroup finds its A rows: contiguous rows of a grouped input, a single group, or rows
// gathered from the token matrix through the dispatch permutation (the permuted copy of the
// activations is then never written).
enum { ROWS_GROUPED = 0, ROWS_SINGLE = 1, ROWS_GATHER = 2 };
// The backward pass's products read rows as ROWS_GROUPED / ROWS_SINGLE do, and take their B operand
// K-major (a weight in its stored layout, e.g. dH = dY W3 with W3 [d, c]); their own values also
// give them their own symbols, so profilers tell them from the forward's launches.
enum { ROWS_GROUPED_BWD = 3, ROWS_SINGLE_BWD = 4 };
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------------------------------------
// M-tile table: tile_start[g] = sum_{g' < g} ceil(count_g' / BM), and tile_group[t] = the group of
// M-tile t (-1 for t >= total, up to max_tiles).  One block, G <= 1024.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_tile_table(const int32_t* __restrict__ offsets, int G, int BM,
                                                     int max_tiles, int32_t* __restrict__ tile_start,
                                                     int32_t* __restrict__ tile_group) {
  __shared__ int32_t s[1024];
  const int t = threadIdx.x;
  int v = 0;
  if (t < G) {
    const int cnt = offsets[t + 1] - offsets[t];
    v = (cnt + BM - 1) / BM;
  }
  s[t] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (t >= off) ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  const int total = s[1023];
  if (t < G) {
    tile_start[t + 1] = s[t];
    for (int j = s[t] - v; j < s[t] && j < max_tiles; ++j) tile_group[j] = t;
  }
  if (t == 0) tile_start[0] = 0;
  for (int j = total + t; j < max_tiles; j += 1024) tile_group[j] = -1;
}

int launch_tile_table(const int32_t* offsets, int G, int BM, int max_tiles, int32_t* tile_start,
                      int32_t* tile_group, hipStream_t s) {
  ProfScope prof(MOE_K_TILE_TABLE, s);
  k_tile_table<<<1, 1024, 0, s>>>(offsets, G, BM, max_tiles, tile_start, tile_group);
  return check_launch("tile table");
}

// ------------------------------------------------------------------------------------------------
// bf16 MFMA tile kernel
// ------------------------------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// K depth of one LDS stage and the number of stages in the ring.  A stage holds BM + BN rows of
// BK bf16 values; two stages of BK = 64 or four of BK = 32 fill 128 KB of the 160 KB LDS.
#ifndef FSM_BK
#define FSM_BK 64
#endif
#ifndef FSM_STAGES
#define FSM_STAGES 2
#endif
constexpr int kBK = FSM_BK, kStages = FSM_STAGES;
static_assert(kBK == 32 || kBK == 64, "BK must be 32 or 64");
static_assert(kStages >= 2 && kStages <= 5, "2 to 5 LDS stages");

// Physical 16-byte chunk of logical chunk c in LDS tile row r.  Rows are BK * 2 bytes; the XOR
// makes the eight rows that one ds_read_b128 group of 8 lanes touches cover all 32 banks.
template <int BK>
__device__ __forceinline__ int lds_swz(int r) { return BK == 64 ? (r & 7) : ((r >> 1) & 3); }

// ROWS (ROWS_GROUPED / ROWS_SINGLE / ROWS_GATHER) also gives routed and shared launches their own
// symbols, so profilers report them separately.
// BNT: B (weight) rows are loaded with the nontemporal hint, for groups that fit in one M-tile, whose
// weight lines no other workgroup reads.
template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, int ROWS, int BK_ = kBK, int S_ = kStages,
          bool BNT = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm_bf16(GemmArgs p) {
  constexpr int NT = 64 * WAVES_M * WAVES_N, NW = NT / 64;
  constexpr int BK = BK_, S = S_;
  constexpr bool PAIRED = EPI == EPI_SWIGLU || EPI == EPI_UG;   // tile holds W1 and W2 columns
  static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
  static_assert(S >= 2 && S <= 5, "2 to 5 LDS stages");
  constexpr int KSL = BK / 32;                 // MFMA K slices per stage
  constexpr int CPR = BK / 8;                  // 16-byte chunks per LDS row
  constexpr int RUN_ROWS = 64 / CPR;           // rows in one wave's 1 KB direct-to-LDS run
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_RUNS = BM / RUN_ROWS / NW, B_RUNS = BN / RUN_ROWS / NW;  // runs per wave per stage
  constexpr int LOADS = A_RUNS + B_RUNS;       // vector-memory operations per wave per stage
  constexpr int STAGE = (BM + BN) * BK;        // bf16 elements per stage (A rows, then B rows)
  static_assert(A_RUNS * RUN_ROWS * NW == BM && B_RUNS * RUN_ROWS * NW == BN, "runs must tile the stage");
  static_assert(!PAIRED || (FN % 2) == 0, "SwiGLU needs paired fragments");
  static_assert(!PAIRED || (BN / 2) % (B_RUNS * RUN_ROWS) == 0, "a wave's B rows must lie in one half");
  static_assert(FM * 16 == WTM && FN * 16 == WTN, "wave tile must be a multiple of 16");
  static_assert(FM >= FN, "the fragment pipeline prefetches one B fragment per A row block");
  static_assert(LOADS * (S - 2) < 64, "vmcnt range");
  // K-major B: a stage's B part is BK rows of BN values (rows of BN * 2 bytes, 16-byte chunks
  // XOR-swizzled by 2 (row mod 4)), and a 16 x 32 fragment is two transposing LDS reads
  // (ds_read_b64_tr_b16), each giving every lane 4 consecutive K values of its column.
  constexpr bool BKM = ROWS == ROWS_GROUPED_BWD || ROWS == ROWS_SINGLE_BWD;
  constexpr int BR = BKM ? 2 : 1;              // LDS reads per B fragment
  static_assert(!BKM || (!PAIRED && BK == 64 && BN == 256), "K-major B: plain products, BK 64, BN 256");

  // one named array per stage, so the compiler can tell the stage being filled from the one read
  __shared__ __attribute__((aligned(16))) uint16_t s0[STAGE], s1[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s2[S > 2 ? STAGE : 8], s3[S > 3 ? STAGE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t s4[S > 4 ? STAGE : 8];

  // the wave index is uniform across the wave: readfirstlane lets the compiler keep it (and every
  // address derived from it) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int mt, nt;
  if (!map_tile(p, BM, mt, nt)) return;

  int g, row0, rows;
  if (!resolve_mtile(p, mt, BM, g, row0, rows)) return;

  const int64_t K = p.K;
  const uint16_t* Ab = static_cast<const uint16_t*>(p.A) + int64_t(row0) * K;
  const uint16_t* Bu;
  const uint16_t* Bg;
  int nvalid;
  if (PAIRED) {
    const int n0 = nt * (BN / 2);
    Bu = static_cast<const uint16_t*>(p.B1) + g * p.b_group_stride + int64_t(n0) * K;
    Bg = static_cast<const uint16_t*>(p.B2) + g * p.b_group_stride + int64_t(n0) * K;
    nvalid = min(BN / 2, p.n_out - n0);
  } else {
    const int n0 = nt * BN;
    Bu = static_cast<const uint16_t*>(p.B1) + g * p.b_group_stride + int64_t(n0) * K;
    Bg = Bu;
    nvalid = min(BN, p.n_out - n0);
  }
  // Rows past `rows` (A) or `nvalid` (B) lie beyond the resource size and load as zeros.  K-major
  // B: the resources are the group's whole B1 rows [0, b_k1) and B2 rows [0, K - b_ksplit).
  const __amdgpu_buffer_rsrc_t rA =
      ROWS == ROWS_GATHER ? make_rsrc(p.A, p.a_rows * K * 2) : make_rsrc(Ab, int64_t(rows) * K * 2);
  const uint16_t* B1g = static_cast<const uint16_t*>(p.B1) + g * p.b_group_stride;
  const uint16_t* B2g = p.B2 ? static_cast<const uint16_t*>(p.B2) + g * p.b_group_stride : B1g;
  const __amdgpu_buffer_rsrc_t rU =
      BKM ? make_rsrc(B1g, p.b_k1 * p.ldb * 2) : make_rsrc(Bu, int64_t(nvalid) * K * 2);
  const __amdgpu_buffer_rsrc_t rG =
      BKM ? make_rsrc(B2g, (K - p.b_ksplit) * p.ldb * 2) : make_rsrc(Bg, int64_t(nvalid) * K * 2);
  const uint32_t ldbB = uint32_t(p.ldb) * 2u;   // K-major B: bytes per B row
  const uint32_t rowB = uint32_t(K) * 2u;  // bytes per row of A and B

  // Direct-to-LDS staging: each wave fills whole 1 KB runs (RUN_ROWS tile rows) of a stage with
  // buffer_load ... lds; lane l writes physical chunk l % CPR of row l / CPR of its run, so it
  // loads logical chunk (l % CPR) ^ swz(row), which reproduces the swizzled layout the fragment
  // reads use (runs start on multiples of 8 or 16 rows, so the swizzle of a run row is that of
  // l / CPR).
  const int d_row = lane / CPR, d_ch = (lane % CPR) ^ lds_swz<BK>(d_row);
  uint32_t dA[A_RUNS], dB[B_RUNS];
  if (ROWS == ROWS_GATHER) {
    // all gather indices are requested before the first is used; rows past the tile read a valid
    // index and are then pointed beyond the resource, so they load zeros
    int src[A_RUNS];
#pragma unroll
    for (int i = 0; i < A_RUNS; ++i) src[i] = p.gather[row0 + min((wave * A_RUNS + i) * RUN_ROWS + d_row, rows - 1)];
#pragma unroll
    for (int i = 0; i < A_RUNS; ++i) {
      const int r = (wave * A_RUNS + i) * RUN_ROWS + d_row;
      dA[i] = r < rows ? uint32_t(src[i] / p.gather_k) * rowB + uint32_t(d_ch) * 16u : 0x80000000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < A_RUNS; ++i) dA[i] = uint32_t((wave * A_RUNS + i) * RUN_ROWS + d_row) * rowB + uint32_t(d_ch) * 16u;
  }
  const int wb_row0 = wave * B_RUNS * RUN_ROWS;  // first B tile row of this wave
  const bool b_gate = PAIRED && wb_row0 >= BN / 2;
  const __amdgpu_buffer_rsrc_t rBw = b_gate ? rG : rU;
#pragma unroll
  for (int i = 0; i < B_RUNS; ++i) {
    if (BKM) {
      // run i of this wave = B rows 2 (wave B_RUNS + i) + {0, 1}; lane l fills physical chunk
      // l % 32 of its row with the logical chunk (l % 32) ^ 2 (row mod 4)
      const int r = 2 * (wave * B_RUNS + i) + (lane >> 5);
      const int lc = (lane & 31) ^ ((2 * r) & 7);
      dB[i] = uint32_t(r) * ldbB + uint32_t(nt * BN) * 2u + uint32_t(lc) * 16u;
    } else {
      const int r = wb_row0 + i * RUN_ROWS + d_row;
      dB[i] = uint32_t(b_gate ? r - BN / 2 : r) * rowB + uint32_t(d_ch) * 16u;
    }
  }


  // Fragment reads: rows (base + 16 i + lane % 16); base is a multiple of 16, so the swizzle
  // term depends on the lane only.
  const int fa0 = (wm * WTM + (lane & 15)) * BK;
  const int fb0 = BM * BK + (PAIRED ? wn * (WTN / 2) : wn * WTN) * BK + (lane & 15) * BK;
  const int sw = lds_swz<BK>(lane & 15);
  // K-major B fragment reads: lane (q = lane / 16, j = lane % 16) reads row 8q + j/4 (+ 4 for the
  // upper half of its K values) at columns 4 (j % 4) .. + 3 of the fragment's 16; the swizzle of
  // those rows is 2 (j / 4)
  const int tr_base = (8 * (lane >> 4) + ((lane & 15) >> 2)) * BN + 4 * (lane & 1);
  const int tr_cb = (wn * WTN) / 8 + ((lane & 3) >> 1), tr_swz = 2 * ((lane & 15) >> 2);

  // A wave whose rows all lie past the group's last row (in the ragged last M-tile of a group)
  // skips its MFMAs and fragment reads: those rows are never stored.  It still loads its share of
  // every stage and meets every barrier.
  const bool live = wm * WTM < rows;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#define FSM_SM(BUF) ((BUF) == 0 ? s0 : (BUF) == 1 ? s1 : (BUF) == 2 ? s2 : (BUF) == 3 ? s3 : s4)
#define FSM_DMA_STAGE(KT, BUF)                                                                     \
  {                                                                                                \
    const uint32_t kb = uint32_t(KT) * BK * 2u;                                                    \
    _Pragma("unroll") for (int i = 0; i < A_RUNS; ++i)                                             \
      FSM_LDS_DMA16(rA, &FSM_SM(BUF)[(wave * A_RUNS + i) * RUN_ROWS * BK], dA[i] + kb);             \
    if (BKM) {                                                                                     \
      const int k0 = (KT) * BK;                                                                    \
      const bool second = p.b_ksplit > 0 && k0 >= p.b_ksplit;                                      \
      const uint32_t kbb = uint32_t(second ? k0 - p.b_ksplit : k0) * ldbB;                         \
      _Pragma("unroll") for (int i = 0; i < B_RUNS; ++i)                                           \
        FSM_LDS_DMA16(second ? rG : rU, &FSM_SM(BUF)[BM * BK + (wave * B_RUNS + i) * 512], dB[i] + kbb); \
    } else {                                                                                       \
      _Pragma("unroll") for (int i = 0; i < B_RUNS; ++i) {                                         \
        if (BNT) FSM_LDS_DMA16_NT(rBw, &FSM_SM(BUF)[BM * BK + (wb_row0 + i * RUN_ROWS) * BK], dB[i] + kb); \
        else FSM_LDS_DMA16(rBw, &FSM_SM(BUF)[BM * BK + (wb_row0 + i * RUN_ROWS) * BK], dB[i] + kb);    \
      }                                                                                            \
    }                                                                                              \
  }
#define FSM_BROW(J) \
  ((PAIRED) ? ((J) < FN / 2 ? (J) * 16 : BN / 2 + ((J) - FN / 2) * 16) : (J) * 16)
#define FSM_LDA(BUF, KS, I) \
  (*reinterpret_cast<const bf16x8*>(&FSM_SM(BUF)[fa0 + (I) * 16 * BK + ((((KS) * 4 + (lane >> 4)) ^ sw) << 3)]))
#define FSM_LDB_TR(BUF, KS, J, H)                                                                \
  __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(              \
      &FSM_SM(BUF)[BM * BK + tr_base + ((KS) * 32 + 4 * (H)) * BN + (((tr_cb + 2 * (J)) ^ tr_swz) << 3)]))
#define FSM_LDB(BUF, KS, J)                                                                        \
  (BKM ? __builtin_bit_cast(bf16x8, __builtin_shufflevector(FSM_LDB_TR(BUF, KS, J, 0),             \
                                                            FSM_LDB_TR(BUF, KS, J, 1), 0, 1, 2, 3, 4, 5, 6, 7)) \
       : *reinterpret_cast<const bf16x8*>(&FSM_SM(BUF)[fb0 + FSM_BROW(J) * BK + ((((KS) * 4 + (lane >> 4)) ^ sw) << 3)]))
  // One stage's MFMAs with the fragment reads software-pipelined: the A fragment for row block
  // i+1 (and, when the stage has a second K slice, that slice's B fragments) are read before the
  // MFMAs of row block i, and scheduling groups pin that order, so an LDS read is always in flight
  // under FN MFMAs instead of being waited for right before its first use.
#define FSM_STEP0(BUF, I, WITH_B)                                                              \
  {                                                                                            \
    a_nxt = ((I) + 1 < FM) ? FSM_LDA(BUF, 0, (I) + 1) : FSM_LDA(BUF, KSL - 1, 0);               \
    if (WITH_B) b1[I] = FSM_LDB(BUF, 1, I);                                                    \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
      acc[I][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[j], a_cur, acc[I][j], 0, 0, 0);   \
    __builtin_amdgcn_sched_group_barrier(0x100, (WITH_B) ? 1 + BR : 1, 0);                     \
    __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                        \
    a_cur = a_nxt;                                                                             \
  }
#define FSM_COMPUTE(BUF)                                                                       \
  {                                                                                            \
    bf16x8 b0[FN], b1[FN], a_cur, a_nxt;                                                       \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) b0[j] = FSM_LDB(BUF, 0, j);                 \
    a_cur = FSM_LDA(BUF, 0, 0);                                                                \
    __builtin_amdgcn_sched_group_barrier(0x100, FN * BR + 1, 0);                               \
    if (KSL == 2) {                                                                            \
      _Pragma("unroll") for (int i = 0; i < FN; ++i) FSM_STEP0(BUF, i, true);                  \
      _Pragma("unroll") for (int i = FN; i < FM; ++i) FSM_STEP0(BUF, i, false);                \
      _Pragma("unroll") for (int i = 0; i < FM - 1; ++i) {                                     \
        a_nxt = FSM_LDA(BUF, 1, i + 1);                                                        \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                         \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[j], a_cur, acc[i][j], 0, 0, 0); \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                    \
        a_cur = a_nxt;                                                                         \
      }                                                                                        \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
        acc[FM - 1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[j], a_cur, acc[FM - 1][j], 0, 0, 0); \
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                      \
    } else {                                                                                   \
      _Pragma("unroll") for (int i = 0; i < FM - 1; ++i) FSM_STEP0(BUF, i, false);             \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
        acc[FM - 1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[j], a_cur, acc[FM - 1][j], 0, 0, 0); \
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);                                      \
      (void)b1;                                                                                \
    }                                                                                          \
  }
  // Workgroup barrier without a memory fence: __syncthreads() would also wait for every
  // outstanding direct-to-LDS load (vmcnt(0)), including the stages still meant to be in flight.
  // The explicit s_waitcnt before it covers this wave's loads of the next stage; every LDS read
  // of the current stage has been consumed by an MFMA before the barrier, so the buffer refilled
  // after it is free.  The empty asm statements keep the compiler from moving memory accesses
  // across the barrier.
#define FSM_BARRIER()                   \
  {                                     \
    asm volatile("" ::: "memory");      \
    __builtin_amdgcn_s_barrier();       \
    asm volatile("" ::: "memory");      \
  }
  // One ring step on stage buffer J: refill the buffer read one step earlier with stage kt+S-1,
  // run this stage's MFMAs, then wait until the next stage is in LDS for every wave.  When fewer
  // than S-2 later stages were issued (the tail), the wait falls back to vmcnt(0).
#define FSM_RING_STEP(J)                                                                       \
  {                                                                                            \
    if (kt + S - 1 < KT) FSM_DMA_STAGE(kt + S - 1, ((J) + S - 1) % S);                         \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    if (live) FSM_COMPUTE(J)                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    if (++kt >= KT) break;                                                                     \
    if (kt + S - 2 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS * (S - 2)));              \
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                                            \
    FSM_BARRIER();                                                                             \
  }

  const int KT = p.K / BK;
  // prologue: stages 0 .. S-2 in flight, then wait for stage 0.  Each branch is straight-line
  // code, so the compiler's own wait-count tracking sees exactly which stages are still pending.
  if (KT >= S - 1) {
#pragma unroll
    for (int st = 0; st < S - 1; ++st) FSM_DMA_STAGE(st, st);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS * (S - 2)));
  } else {
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < KT) FSM_DMA_STAGE(st, st);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  FSM_BARRIER();
  // unrolled S times so that every step names its stage buffers as constants
  for (int kt = 0;;) {
    FSM_RING_STEP(0);
    FSM_RING_STEP(1);
    if (S > 2) FSM_RING_STEP(2 % S);
    if (S > 3) FSM_RING_STEP(3 % S);
    if (S > 4) FSM_RING_STEP(4 % S);
  }
#undef FSM_RING_STEP
#undef FSM_BARRIER
#undef FSM_DMA_STAGE
#undef FSM_BROW
#undef FSM_LDA
#undef FSM_LDB
#undef FSM_LDB_TR
#undef FSM_SM
#undef FSM_STEP0
#undef FSM_COMPUTE

  // epilogue: lane holds rows m = .. + (lane & 15), columns n = .. + 4*(lane >> 4) + {0..3}.
  // Where the tile's columns all lie below n_out (every tile but a ragged last N-tile), the bf16
  // epilogues pair adjacent fragments into 16-byte stores (pair_words); partner lanes share their
  // row, so they skip or store it together.
  const int ml = lane & 15, nl = (lane >> 4) * 4, pc = pair_col(lane);
  constexpr int TILE_N = PAIRED ? BN / 2 : BN;
  const bool full_n = (FN / (PAIRED ? 2 : 1)) % 2 == 0 && (nt + 1) * TILE_N <= p.n_out;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = wm * WTM + i * 16 + ml;
    if (m >= rows) continue;
    const int64_t orow = int64_t(row0 + m);
    if (EPI == EPI_SWIGLU && full_n) {
      uint16_t* out = static_cast<uint16_t*>(p.out) + orow * p.n_out + nt * (BN / 2) + wn * (WTN / 2) + pc;
#pragma unroll
      for (int j = 0; j + 1 < FN / 2; j += 2) {
        const f32x4 u0 = acc[i][j], g0 = acc[i][j + FN / 2], u1 = acc[i][j + 1], g1 = acc[i][j + 1 + FN / 2];
        *reinterpret_cast<st_u32x4*>(out + j * 16) =
            pair_words(pack2(u0[0] * silu_f(g0[0]), u0[1] * silu_f(g0[1])), pack2(u0[2] * silu_f(g0[2]), u0[3] * silu_f(g0[3])),
                       pack2(u1[0] * silu_f(g1[0]), u1[1] * silu_f(g1[1])), pack2(u1[2] * silu_f(g1[2]), u1[3] * silu_f(g1[3])));
      }
    } else if (EPI == EPI_SWIGLU) {
      uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int col = nt * (BN / 2) + wn * (WTN / 2) + j * 16 + nl;
        if (col >= p.n_out) continue;
        const f32x4 u = acc[i][j], gt = acc[i][j + FN / 2];
        uint2 v;
        v.x = pack2(u[0] * silu_f(gt[0]), u[1] * silu_f(gt[1]));
        v.y = pack2(u[2] * silu_f(gt[2]), u[3] * silu_f(gt[3]));
        *reinterpret_cast<uint2*>(out + orow * p.n_out + col) = v;
      }
    } else if (EPI == EPI_UG && full_n) {
      const int64_t ld = 2 * int64_t(p.n_out);
      uint16_t* out = static_cast<uint16_t*>(p.out) + orow * ld + nt * (BN / 2) + wn * (WTN / 2) + pc;
#pragma unroll
      for (int j = 0; j + 1 < FN / 2; j += 2) {
        const f32x4 u0 = acc[i][j], g0 = acc[i][j + FN / 2], u1 = acc[i][j + 1], g1 = acc[i][j + 1 + FN / 2];
        *reinterpret_cast<st_u32x4*>(out + j * 16) =
            pair_words(pack2(u0[0], u0[1]), pack2(u0[2], u0[3]), pack2(u1[0], u1[1]), pack2(u1[2], u1[3]));
        *reinterpret_cast<st_u32x4*>(out + p.n_out + j * 16) =
            pair_words(pack2(g0[0], g0[1]), pack2(g0[2], g0[3]), pack2(g1[0], g1[1]), pack2(g1[2], g1[3]));
      }
    } else if (EPI == EPI_UG) {
      uint16_t* out = static_cast<uint16_t*>(p.out);
      const int64_t ld = 2 * int64_t(p.n_out);
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int col = nt * (BN / 2) + wn * (WTN / 2) + j * 16 + nl;
        if (col >= p.n_out) continue;
        const f32x4 u = acc[i][j], gt = acc[i][j + FN / 2];
        *reinterpret_cast<uint2*>(out + orow * ld + col) = make_uint2(pack2(u[0], u[1]), pack2(u[2], u[3]));
        *reinterpret_cast<uint2*>(out + orow * ld + p.n_out + col) = make_uint2(pack2(gt[0], gt[1]), pack2(gt[2], gt[3]));
      }
    } else if (EPI == EPI_PLAIN && full_n) {
      uint16_t* out = static_cast<uint16_t*>(p.out) + orow * p.n_out + nt * BN + wn * WTN + pc;
#pragma unroll
      for (int j = 0; j + 1 < FN; j += 2) {
        const f32x4 a = acc[i][j], b = acc[i][j + 1];
        *reinterpret_cast<st_u32x4*>(out + j * 16) =
            pair_words(pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]), pack2(b[2], b[3]));
      }
    } else if (EPI == EPI_PLAIN) {
      uint16_t* out = static_cast<uint16_t*>(p.out);
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
    } else {
      float* out = static_cast<float*>(p.out);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = nt * BN + wn * WTN + j * 16 + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (col + r < p.n_out) {
            const float b = p.bias ? p.bias[col + r] : 0.f;
            out[orow * p.n_out + col + r] = acc[i][j][r] + b;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// float32 path (the tiny fp32 workload): 16 x 16 output tile per workgroup, plain FMA.
// ------------------------------------------------------------------------------------------------
template <int EPI, int ROWS>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs p) {
  constexpr int BM = 16, BN = 16, BKF = 16;
  __shared__ float sA[BM][BKF + 1], sU[BN][BKF + 1], sG[BN][BKF + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int mt = blockIdx.x / p.n_tiles, nt = blockIdx.x % p.n_tiles;

  int g, row0, rows;
  if (!resolve_mtile(p, mt, BM, g, row0, rows)) return;
  const int K = p.K;
  const int n0 = nt * BN;
  const float* A = static_cast<const float*>(p.A) + int64_t(row0) * K;
  const float* B1 = static_cast<const float*>(p.B1) + g * p.b_group_stride;
  const float* B2 = (EPI == EPI_SWIGLU) ? static_cast<const float*>(p.B2) + g * p.b_group_stride : nullptr;

  float accU = 0.f, accG = 0.f;
  for (int k0 = 0; k0 < K; k0 += BKF) {
    const int k = k0 + tx;
    if (ROWS == ROWS_GATHER)
      sA[ty][tx] = (ty < rows && k < K)
                       ? static_cast<const float*>(p.A)[int64_t(p.gather[row0 + ty] / p.gather_k) * K + k]
                       : 0.f;
    else
      sA[ty][tx] = (ty < rows && k < K) ? A[int64_t(ty) * K + k] : 0.f;
    const int n = n0 + ty;
    const bool nok = n < p.n_out && k < K;
    sU[ty][tx] = nok ? B1[int64_t(n) * K + k] : 0.f;
    if (EPI == EPI_SWIGLU) sG[ty][tx] = nok ? B2[int64_t(n) * K + k] : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk) {
      accU = fmaf(sA[ty][kk], sU[tx][kk], accU);
      if (EPI == EPI_SWIGLU) accG = fmaf(sA[ty][kk], sG[tx][kk], accG);
    }
    __syncthreads();
  }
  const int n = n0 + tx;
  if (ty >= rows || n >= p.n_out) return;
  float* out = static_cast<float*>(p.out);
  const int64_t o = int64_t(row0 + ty) * p.n_out + n;
  if (EPI == EPI_SWIGLU) {
    out[o] = accU * (accG / (1.0f + expf(-accG)));
  } else if (EPI == EPI_F32_BIAS) {
    out[o] = accU + (p.bias ? p.bias[n] : 0.f);
  } else {
    out[o] = accU;
  }
}

// ------------------------------------------------------------------------------------------------
// host launchers
// ------------------------------------------------------------------------------------------------
namespace {
// bf16 tilings (the phase-1 tile holds BN/2 columns of W1 and the same BN/2 columns of W2)
#ifndef FSM_P1
#define FSM_P1 256, 256, 2, 4, 4   /* BM, BN, waves along M, waves along N, M-tiles per group */
#endif
#ifndef FSM_P2
#define FSM_P2 256, 256, 2, 4, 4
#endif
#ifndef FSM_R
#define FSM_R 256, 256, 2, 4, 1
#endif
struct TileCfg { int bm, bn, wm, wn, gm; int bk = kBK; int st = kStages; };
constexpr TileCfg kP1{FSM_P1}, kP2{FSM_P2}, kR{FSM_R};
// Groups of a few dozen rows (a decode batch spread over all experts: 32 rows per expert for 1024
// tokens, k = 8, E = 256) would leave most of a 256-row tile empty; there the product is bound by
// the weight stream, not by the MFMA, and 64-row tiles (4 waves of 64 x 64) keep the padding
// small.  They are used when the groups average at most kSmallRows rows, or when 256-row tiles
// would not give every CU a workgroup (the shared expert of a decode batch: 1024 rows, one
// group).  Three 40 KB stages (one workgroup per CU, two stages in flight) stream the weights
// 1.5% faster in the decode stack than two.
#ifndef FSM_SMALL_STAGE
#define FSM_SMALL_STAGE 64, 3
#endif
constexpr TileCfg kS1{64, 256, 1, 4, 4, FSM_SMALL_STAGE}, kS2{64, 256, 1, 4, 4, FSM_SMALL_STAGE};
constexpr int kSmallRows = 96, kCus = 256;
constexpr int R_BM = kR.bm, R_BN = kR.bn, R_WM = kR.wm, R_WN = kR.wn;
// Router of a small batch (a decode step): 256 x 256 tiles would give a 1024-token batch four
// workgroups; 64 x 64 tiles (4 waves of 64 x 16) give it 64.
constexpr TileCfg kRS{64, 64, 1, 4, 1};
constexpr int F_BM = 16, F_BN = 16;

bool small_tiles(int64_t N, int32_t G, int64_t c, int dtype) {
  if (dtype != MOE_BF16) return false;
  const int64_t big_grid = (cdiv(N, kP1.bm) + G) * cdiv(c, kP1.bn / 2);
  return N <= int64_t(kSmallRows) * G || big_grid < kCus;
}

// M-tile rows of the two phases for this problem
void tile_rows(int64_t N, int32_t G, int64_t c, int dtype, int& bm1, int& bm2) {
  if (dtype != MOE_BF16) {
    bm1 = bm2 = F_BM;
  } else if (small_tiles(N, G, c, dtype)) {
    bm1 = kS1.bm;
    bm2 = kS2.bm;
  } else {
    bm1 = kP1.bm;
    bm2 = kP2.bm;
  }
}

// Both phases of the bf16 grouped product with tile configurations C1 (gate/up) and C2 (down).
// stream_b: the routed launches load their weights with the nontemporal hint (64-row tiles only).
template <const TileCfg& C1, const TileCfg& C2>
int launch_bf16_pair(GemmArgs& a1, GemmArgs& a2, int rows1, int rows2, int64_t mt1, int64_t mt2, int64_t c,
                     int64_t d, int32_t G, hipStream_t s, hipEvent_t mid, const int* kinds, bool stream_b) {
  constexpr bool kSmall = C1.bm == kS1.bm && C2.bm == kS2.bm;
  stream_b = stream_b && kSmall;
  a1.group_m = C1.gm;
  a1.n_tiles = int32_t(cdiv(c, C1.bn / 2));
  a1.quad_nb = quad_width(a1.n_tiles, a1.group_m);
  const dim3 grid1(unsigned(quad_grid(mt1, a1.n_tiles, a1.group_m, a1.quad_nb)));
  constexpr int nt1 = 64 * C1.wm * C1.wn;
  {
    ProfScope prof(kinds ? kinds[0] : G > 1 ? MOE_K_GEMM_GATE_UP : MOE_K_DENSE_GATE_UP, s);
    if (rows1 == ROWS_GATHER && stream_b)
      k_gemm_bf16<C1.bm, C1.bn, C1.wm, C1.wn, EPI_SWIGLU, ROWS_GATHER, C1.bk, C1.st, kSmall><<<grid1, nt1, 0, s>>>(a1);
    else if (rows1 == ROWS_GATHER)
      k_gemm_bf16<C1.bm, C1.bn, C1.wm, C1.wn, EPI_SWIGLU, ROWS_GATHER, C1.bk, C1.st><<<grid1, nt1, 0, s>>>(a1);
    else if (rows1 == ROWS_GROUPED && stream_b)
      k_gemm_bf16<C1.bm, C1.bn, C1.wm, C1.wn, EPI_SWIGLU, ROWS_GROUPED, C1.bk, C1.st, kSmall><<<grid1, nt1, 0, s>>>(a1);
    else if (rows1 == ROWS_GROUPED)
      k_gemm_bf16<C1.bm, C1.bn, C1.wm, C1.wn, EPI_SWIGLU, ROWS_GROUPED, C1.bk, C1.st><<<grid1, nt1, 0, s>>>(a1);
    else
      k_gemm_bf16<C1.bm, C1.bn, C1.wm, C1.wn, EPI_SWIGLU, ROWS_SINGLE, C1.bk, C1.st><<<grid1, nt1, 0, s>>>(a1);
    if (int rc = check_launch("grouped gemm phase 1")) return rc;
  }
  if (mid) {
    const hipError_t e = hipEventRecord(mid, s);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  a2.group_m = C2.gm;
  a2.n_tiles = int32_t(cdiv(d, C2.bn));
  a2.quad_nb = quad_width(a2.n_tiles, a2.group_m);
  const dim3 grid2(unsigned(quad_grid(mt2, a2.n_tiles, a2.group_m, a2.quad_nb)));
  constexpr int nt2 = 64 * C2.wm * C2.wn;
  ProfScope prof(kinds ? kinds[1] : G > 1 ? MOE_K_GEMM_DOWN : MOE_K_DENSE_DOWN, s);
  if (rows2 == ROWS_GROUPED && stream_b)
    k_gemm_bf16<C2.bm, C2.bn, C2.wm, C2.wn, EPI_PLAIN, ROWS_GROUPED, C2.bk, C2.st, kSmall><<<grid2, nt2, 0, s>>>(a2);
  else if (rows2 == ROWS_GROUPED)
    k_gemm_bf16<C2.bm, C2.bn, C2.wm, C2.wn, EPI_PLAIN, ROWS_GROUPED, C2.bk, C2.st><<<grid2, nt2, 0, s>>>(a2);
  else
    k_gemm_bf16<C2.bm, C2.bn, C2.wm, C2.wn, EPI_PLAIN, ROWS_SINGLE, C2.bk, C2.st><<<grid2, nt2, 0, s>>>(a2);
  return check_launch("grouped gemm phase 2");
}

struct SwigluWs {
  int32_t* ts1;
  int32_t* grp1;
  int32_t* ts2;
  int32_t* grp2;
  void* H;
};

SwigluWs carve(void* ws, int32_t G, int64_t N, int64_t c, int dtype, size_t* total) {
  const size_t esz = dtype == MOE_BF16 ? 2 : 4;
  int bm1, bm2;
  tile_rows(N, G, c, dtype, bm1, bm2);
  const int64_t mt1 = cdiv(N, bm1) + G, mt2 = cdiv(N, bm2) + G;
  size_t off = 0;
  SwigluWs w;
  char* base = static_cast<char*>(ws);
  w.ts1 = reinterpret_cast<int32_t*>(base + off);
  off = align_up(off + size_t(G + 1) * 4, 256);
  w.grp1 = reinterpret_cast<int32_t*>(base + off);
  off = align_up(off + size_t(mt1) * 4, 256);
  w.ts2 = reinterpret_cast<int32_t*>(base + off);
  off = align_up(off + size_t(G + 1) * 4, 256);
  w.grp2 = reinterpret_cast<int32_t*>(base + off);
  off = align_up(off + size_t(mt2) * 4, 256);
  w.H = base + off;
  off = align_up(off + size_t(N) * size_t(c) * esz, 256);
  if (total) *total = off;
  return w;
}
}  // namespace

size_t swiglu_ws_bytes(int64_t N, int32_t G, int64_t c, int dtype) {
  size_t total = 0;
  carve(nullptr, G, N, c, dtype, &total);
  return total;
}

int launch_grouped_swiglu(const void* X, const int32_t* offsets, int32_t G, const void* W1,
                          const void* W2, const void* W3, int dtype, int64_t N, int64_t d, int64_t c,
                          void* Y, void* ws, hipStream_t s, const int32_t* gather, int32_t gather_k,
                          int64_t x_rows, hipEvent_t mid, const int* kinds) {
  SwigluWs w = carve(ws, G, N, c, dtype, nullptr);
  if (N == 0) {   // nothing to compute; the phase event still marks this point of the stream
    const hipError_t e = mid ? hipEventRecord(mid, s) : hipSuccess;
    return e == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  const bool bf = dtype == MOE_BF16;
  int bm1, bm2;
  tile_rows(N, G, c, dtype, bm1, bm2);
  const int64_t mt1 = cdiv(N, bm1) + G, mt2 = cdiv(N, bm2) + G;
  {
    ProfScope prof(MOE_K_TILE_TABLE, s);
    k_tile_table<<<1, 1024, 0, s>>>(offsets, G, bm1, int(mt1), w.ts1, w.grp1);
    if (int rc = check_launch("tile table")) return rc;
  }
  if (bm2 != bm1) {
    ProfScope prof(MOE_K_TILE_TABLE, s);
    k_tile_table<<<1, 1024, 0, s>>>(offsets, G, bm2, int(mt2), w.ts2, w.grp2);
    if (int rc = check_launch("tile table")) return rc;
  } else {
    w.ts2 = w.ts1;
    w.grp2 = w.grp1;
  }

  GemmArgs a1{};
  a1.A = X; a1.B1 = W1; a1.B2 = W2; a1.out = w.H; a1.bias = nullptr;
  a1.offsets = offsets; a1.tile_start = w.ts1; a1.tile_group = w.grp1; a1.b_group_stride = c * d;
  a1.K = int32_t(d); a1.n_out = int32_t(c); a1.M = int32_t(N); a1.G = G; a1.group_m = 1;
  a1.gather = gather; a1.gather_k = gather_k; a1.a_rows = x_rows;

  GemmArgs a2{};
  a2.A = w.H; a2.B1 = W3; a2.B2 = nullptr; a2.out = Y; a2.bias = nullptr;
  a2.offsets = offsets; a2.tile_start = w.ts2; a2.tile_group = w.grp2; a2.b_group_stride = d * c;
  a2.K = int32_t(c); a2.n_out = int32_t(d); a2.M = int32_t(N); a2.G = G; a2.group_m = 1;

  const int rows1 = gather ? ROWS_GATHER : (G > 1 ? ROWS_GROUPED : ROWS_SINGLE);
  const int rows2 = G > 1 ? ROWS_GROUPED : ROWS_SINGLE;
  // Routed groups that average at most one 64-row tile: each expert's weights are read by one M-tile
  // per N-tile, so they stream past the caches (the shared expert's weights are reused by every
  // M-tile and keep the default policy).
  const bool stream_b = G > 1 && N <= int64_t(kS1.bm) * G;
  if (bf && small_tiles(N, G, c, dtype))
    return launch_bf16_pair<kS1, kS2>(a1, a2, rows1, rows2, mt1, mt2, c, d, G, s, mid, kinds, stream_b);
  if (bf) return launch_bf16_pair<kP1, kP2>(a1, a2, rows1, rows2, mt1, mt2, c, d, G, s, mid, kinds, false);
  a1.n_tiles = int32_t(cdiv(c, F_BN));
  {
    ProfScope prof(kinds ? kinds[0] : G > 1 ? MOE_K_GEMM_GATE_UP : MOE_K_DENSE_GATE_UP, s);
    if (rows1 == ROWS_GATHER)
      k_gemm_f32<EPI_SWIGLU, ROWS_GATHER><<<dim3(unsigned(mt1 * a1.n_tiles)), 256, 0, s>>>(a1);
    else
      k_gemm_f32<EPI_SWIGLU, ROWS_GROUPED><<<dim3(unsigned(mt1 * a1.n_tiles)), 256, 0, s>>>(a1);
    if (int rc = check_launch("grouped gemm phase 1 (f32)")) return rc;
  }
  if (mid) {
    const hipError_t e = hipEventRecord(mid, s);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  a2.n_tiles = int32_t(cdiv(d, F_BN));
  ProfScope prof(kinds ? kinds[1] : G > 1 ? MOE_K_GEMM_DOWN : MOE_K_DENSE_DOWN, s);
  k_gemm_f32<EPI_PLAIN, ROWS_GROUPED><<<dim3(unsigned(mt2 * a2.n_tiles)), 256, 0, s>>>(a2);
  return check_launch("grouped gemm phase 2 (f32)");
}

int launch_router_logits(const void* A, const void* W_R, const float* bias, int dtype, int64_t T,
                         int64_t d, int32_t E, float* logits, hipStream_t s) {
  if (T == 0) return MOE_OK;
  GemmArgs a{};
  a.A = A; a.B1 = W_R; a.B2 = nullptr; a.out = logits; a.bias = bias;
  a.offsets = nullptr; a.tile_start = nullptr; a.tile_group = nullptr; a.b_group_stride = 0;
  a.K = int32_t(d); a.n_out = E; a.M = int32_t(T); a.G = 1; a.group_m = kR.gm;
  ProfScope prof(MOE_K_ROUTER_GEMM, s);
  if (dtype == MOE_BF16) {
    if (cdiv(T, R_BM) * cdiv(E, R_BN) < kCus) {
      a.n_tiles = int32_t(cdiv(E, kRS.bn));
      const int64_t grid = cdiv(T, kRS.bm) * a.n_tiles;
      k_gemm_bf16<kRS.bm, kRS.bn, kRS.wm, kRS.wn, EPI_F32_BIAS, ROWS_SINGLE>
          <<<dim3(unsigned(grid)), 64 * kRS.wm * kRS.wn, 0, s>>>(a);
      return check_launch("router gemm");
    }
    a.n_tiles = int32_t(cdiv(E, R_BN));
    const int64_t grid = cdiv(T, R_BM) * a.n_tiles;
    k_gemm_bf16<R_BM, R_BN, R_WM, R_WN, EPI_F32_BIAS, ROWS_SINGLE><<<dim3(unsigned(grid)), 64 * R_WM * R_WN, 0, s>>>(a);
    return check_launch("router gemm");
  }
  a.n_tiles = int32_t(cdiv(E, F_BN));
  k_gemm_f32<EPI_F32_BIAS, ROWS_GROUPED><<<dim3(unsigned(cdiv(T, F_BM) * a.n_tiles)), 256, 0, s>>>(a);
  return check_launch("router gemm (f32)");
}

// One bf16 product on 256 x 256 tiles for the backward pass: out = X B^T per group (B = B1 + g *
// b_stride, [n_out, K]).  epi EPI_UG: B1 and B2 side by side, out [N, 2 n_out] = (X B1^T | X B2^T);
// EPI_PLAIN: bf16 out [N, n_out]; EPI_F32_BIAS (one group, no bias): fp32 out [N, n_out].  ts / grp:
// the group tile table for 256-row tiles (null with one group).
int launch_bf16_product(int epi, const void* X, const int32_t* offsets, const int32_t* ts, const int32_t* grp,
                        int32_t G, const void* B1, const void* B2, int64_t b_stride, int64_t ldb, int64_t b_k1,
                        int64_t b_ksplit, int64_t N, int64_t K, int64_t n_out, void* out, hipStream_t s,
                        const int32_t* gather, int32_t gather_k, int64_t x_rows, int prof_kind) {
  if (N == 0) return MOE_OK;
  constexpr TileCfg C = kP1;
  if (epi != EPI_UG) {   // K-major B: 32-bit buffer offsets within one group's B1 / B2
    if (ldb < n_out || b_k1 > K || b_ksplit < 0 || b_ksplit % C.bk != 0 || K % C.bk != 0 ||
        (b_ksplit > 0 && !B2) || (b_k1 > K - b_ksplit ? b_k1 : K - b_ksplit) * ldb * 2 >= (int64_t(1) << 31))
      return fail(MOE_ERR_UNSUPPORTED, "backward product: B layout out of range");
  }
  GemmArgs a{};
  a.A = X; a.B1 = B1; a.B2 = B2; a.out = out; a.bias = nullptr;
  a.offsets = offsets; a.tile_start = ts; a.tile_group = grp; a.b_group_stride = b_stride;
  a.K = int32_t(K); a.n_out = int32_t(n_out); a.M = int32_t(N); a.G = G; a.group_m = C.gm;
  a.gather = gather; a.gather_k = gather_k; a.a_rows = x_rows;
  a.ldb = ldb; a.b_k1 = b_k1; a.b_ksplit = int32_t(b_ksplit);
  a.n_tiles = int32_t(cdiv(n_out, epi == EPI_UG ? C.bn / 2 : C.bn));
  a.quad_nb = quad_width(a.n_tiles, a.group_m);
  const int64_t mt = grp ? cdiv(N, C.bm) + G : cdiv(N, C.bm);
  const dim3 grid(unsigned(quad_grid(mt, a.n_tiles, a.group_m, a.quad_nb)));
  constexpr int nt = 64 * C.wm * C.wn;
  ProfScope prof(prof_kind, s);
  if (epi == EPI_UG && gather)
    k_gemm_bf16<C.bm, C.bn, C.wm, C.wn, EPI_UG, ROWS_GATHER, C.bk, C.st><<<grid, nt, 0, s>>>(a);
  else if (epi == EPI_UG)
    k_gemm_bf16<C.bm, C.bn, C.wm, C.wn, EPI_UG, ROWS_SINGLE, C.bk, C.st><<<grid, nt, 0, s>>>(a);
  else if (epi == EPI_PLAIN && grp)
    k_gemm_bf16<C.bm, C.bn, C.wm, C.wn, EPI_PLAIN, ROWS_GROUPED_BWD, C.bk, C.st><<<grid, nt, 0, s>>>(a);
  else if (epi == EPI_PLAIN)
    k_gemm_bf16<C.bm, C.bn, C.wm, C.wn, EPI_PLAIN, ROWS_SINGLE_BWD, C.bk, C.st><<<grid, nt, 0, s>>>(a);
  else
    k_gemm_bf16<C.bm, C.bn, C.wm, C.wn, EPI_F32_BIAS, ROWS_SINGLE_BWD, C.bk, C.st><<<grid, nt, 0, s>>>(a);
  return check_launch("backward product");
}

}  // namespace fsm
