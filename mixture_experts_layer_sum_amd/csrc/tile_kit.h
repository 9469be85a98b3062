// Tile scheduling and direct-to-LDS staging shared by the bf16 and the MXFP8 grouped products.
#pragma once

#include "common.h"

namespace fsm {

constexpr int kBufDword3 = 0x00020000;  // gfx9-family raw buffer descriptor word 3

// 16-byte direct-to-LDS buffer load (device pass only; the host pass needs just the launch stubs
// and never sees the builtin).
//
// The LDS address goes through an empty asm statement, so the compiler cannot tie the load to the
// stage array it fills.  Its own wait-count pass then leaves LDS reads of the other stages alone
// (it otherwise waits for every stage in flight before reading any one); the kernel waits for the
// stage it reads itself, with an explicit s_waitcnt and a barrier.
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, const void* lds, uint32_t voff) {
  uint32_t a = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  asm volatile("" : "+s"(a));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)uintptr_t(a), 16, voff, 0, 0, 0);
}
// 4-byte form (lane l writes LDS bytes 4l .. 4l + 3 of the run)
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rsrc, const void* lds, uint32_t voff) {
  uint32_t a = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  asm volatile("" : "+s"(a));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)uintptr_t(a), 4, voff, 0, 0, 0);
}
// The same 16-byte load with the nontemporal hint (nt): for operand lines that no other workgroup
// reads again (the weights of a group that fits in one M-tile), which then need not displace lines
// that are reused.  A plain stream of such loads from HBM runs 6.9-7.2 TB/s against 6.1-6.3 TB/s
// without the hint (measured on MI355X).
__device__ __forceinline__ void lds_dma16_nt(__amdgpu_buffer_rsrc_t rsrc, const void* lds, uint32_t voff) {
  uint32_t a = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  asm volatile("" : "+s"(a));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)uintptr_t(a), 16, voff, 0, 0, 2);
}
#define FSM_LDS_DMA16(RSRC, LDS, VOFF) lds_dma16((RSRC), (LDS), (VOFF))
#define FSM_LDS_DMA16_NT(RSRC, LDS, VOFF) lds_dma16_nt((RSRC), (LDS), (VOFF))
#define FSM_LDS_DMA4(RSRC, LDS, VOFF) lds_dma4((RSRC), (LDS), (VOFF))
#else
#define FSM_LDS_DMA16(RSRC, LDS, VOFF) ((void)(RSRC), (void)(LDS), (void)(VOFF))
#define FSM_LDS_DMA16_NT(RSRC, LDS, VOFF) ((void)(RSRC), (void)(LDS), (void)(VOFF))
#define FSM_LDS_DMA4(RSRC, LDS, VOFF) ((void)(RSRC), (void)(LDS), (void)(VOFF))
#endif

// 16-byte output stores.  A product issued with the weight fragment first leaves lane group
// q = lane / 16 holding columns 4q .. 4q + 3 of each 16-column fragment (as packed bf16 pairs, two
// dwords).  For two adjacent fragments a (columns 0-15) and b (16-31), one gfx950 permlane16 swap
// per dword trades b's words in groups 0 and 2 for a's words in groups 1 and 3 (the lanes it pairs,
// l and l + 16, hold the same row).  Each lane then holds 8 consecutive columns, starting at
// pair_col(lane) of the 32, and one 16-byte store per lane replaces two 8-byte stores: measured on
// the routed down product, 5% faster, with the same bytes written.
typedef unsigned int st_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int pair_col(int lane) { return ((lane >> 4) & 1) * 16 + (lane >> 5) * 8; }
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ st_u32x4 pair_words(uint32_t a01, uint32_t a23, uint32_t b01, uint32_t b23) {
  const auto s0 = __builtin_amdgcn_permlane16_swap(a01, b01, false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(a23, b23, false, false);
  st_u32x4 v;
  v[0] = s0[0];
  v[1] = s1[0];
  v[2] = s0[1];
  v[3] = s1[1];
  return v;
}
#else
__device__ __forceinline__ st_u32x4 pair_words(uint32_t, uint32_t, uint32_t, uint32_t) { return st_u32x4{}; }
#endif

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave are
// outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufDword3);
}

// Resolve M-tile mt of a grouped product (or of a dense one with M rows) to (group, first row,
// row count).  Returns false for a surplus workgroup.
template <class Args>
__device__ __forceinline__ bool resolve_mtile(const Args& p, int mt, int BM, int& g, int& row0,
                                              int& rows) {
  if (p.tile_group) {
    g = p.tile_group[mt];
    if (g < 0) return false;
    row0 = p.offsets[g] + (mt - p.tile_start[g]) * BM;
    rows = min(BM, p.offsets[g + 1] - row0);
    return true;
  }
  g = 0;
  row0 = mt * BM;
  if (row0 >= p.M) return false;
  rows = min(BM, p.M - row0);
  return true;
}

// Workgroup -> (M-tile, N-tile).  Workgroups are dealt round-robin to the 8 XCDs, so workgroup b
// runs on XCD b % 8 as that XCD's (b / 8)-th workgroup.  Two orders are used; in both, the
// workgroups without a tile (the worst-case grid's surplus) exit at once.
//  - quad_nb > 0 (grouped and shared-expert products): each XCD works through blocks of
//    group_m x quad_nb tiles, about one tile per CU, so the tiles resident on an XCD share
//    activation rows and weight panels in its L2; see quad_grid for the block order.
//  - quad_nb == 0 (router): each XCD is given one contiguous range of the logical tile order, in
//    which group_m M-tiles sweep the N-tiles together.
constexpr int kXcds = 8;

// XCD blocks of group_m x quad_nb tiles (one block per XCD at a time), ordered in 2 x 2 quads:
// the four XCDs that run one quad at the same time pair up on M-groups (same activation rows)
// and on N-blocks (same weight panels), so each line they share is fetched from HBM once and
// found in the memory-side cache by the other XCD.  Blocks go by pairs of M-groups; within a
// pair, the quads of each pair of N-blocks, then (when the N-block count is odd) the last
// N-block's two blocks, so that no block position is left without a tile.  Returns the number
// of workgroups to launch for at most max_mt M-tiles.
inline int64_t quad_grid(int64_t max_mt, int n_tiles, int group_m, int quad_nb) {
  const int64_t n_mg = (max_mt + group_m - 1) / group_m, n_nb = (n_tiles + quad_nb - 1) / quad_nb;
  const int64_t blocks = ((n_mg + 1) / 2) * 2 * n_nb;
  const int64_t rounds = (blocks + kXcds - 1) / kXcds;
  return rounds * kXcds * int64_t(group_m) * quad_nb;
}

template <class Args>
__device__ __forceinline__ bool map_tile(const Args& p, int BM, int& mt, int& nt) {
  const int total_mt = p.tile_group ? p.tile_start[p.G] : (p.M + BM - 1) / BM;
  const int b = blockIdx.x;
  if (p.quad_nb > 0) {
    const int blk_tiles = p.group_m * p.quad_nb;
    const int x = b % kXcds, i = b / kXcds;
    const int blk = (i / blk_tiles) * kXcds + x, pos = i % blk_tiles;
    const int n_nb = (p.n_tiles + p.quad_nb - 1) / p.quad_nb, pairs = n_nb / 2;
    const int row = blk / (2 * n_nb), at = blk % (2 * n_nb);   // M-group pair, block within it
    int mg, nb;
    if (at < 4 * pairs) {   // quad at / 4: M-groups 2 row + {0, 1} x N-blocks 2 (at / 4) + {0, 1}
      mg = 2 * row + (at & 1);
      nb = 2 * (at >> 2) + ((at >> 1) & 1);
    } else {                // the odd last N-block: M-groups 2 row + {0, 1}
      mg = 2 * row + (at - 4 * pairs);
      nb = n_nb - 1;
    }
    mt = mg * p.group_m + pos % p.group_m;
    nt = nb * p.quad_nb + pos / p.group_m;
    return mt < total_mt && nt < p.n_tiles && nt < (nb + 1) * p.quad_nb;
  }
  const int total = total_mt * p.n_tiles;
  if (b >= total) return false;
  const int q = total / kXcds, r = total % kXcds, x = b % kXcds, i = b / kXcds;
  const int L = x * q + min(x, r) + i;
  const int gsz = p.group_m * p.n_tiles;
  const int grp = L / gsz, within = L - grp * gsz;
  const int m_in = min(p.group_m, total_mt - grp * p.group_m);
  mt = grp * p.group_m + within % m_in;
  nt = within / m_in;
  return true;
}

// N-tiles per XCD block of the quad order: one XCD runs 32 tiles at a time (one per CU), so a
// block is group_m x (32 / group_m) tiles, narrowed to a divisor of n_tiles where one is close
// (7 for the 28 N-tiles of a 7168-wide down product) so that no block is ragged.
inline int quad_width(int n_tiles, int group_m) {
  const int target = 32 / group_m;
  for (int q = target; q * 2 > target; --q)
    if (n_tiles % q == 0) return q;
  return target;
}

}  // namespace fsm
