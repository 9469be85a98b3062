// Dispatch permutation for gfx950 ("FarSkip-Collective" section 2.1: the token rows A[l,:] are
// grouped by their selected experts by permuting A).
//
// Every flat slot f = t*k + i is one row.  Rows are ordered by expert, and inside an expert by f
// (a stable counting sort), so the result is unique and deterministic:
//   1. k_perm_hist   per chunk of PCH slots, an LDS histogram of expert ids (integer atomics in
//                    LDS; the counts do not depend on their order)
//   2. k_perm_scan   per expert, the exclusive prefix of the chunk counts over chunks, and the
//                    exclusive prefix of the expert totals over experts (= expert offsets)
//   3. k_perm_rank   each chunk walks its slots in rounds of 256 in slot order; inside a round a
//                    slot's rank among equal experts comes from wavefront ballots over the bits
//                    of the expert id (the lanes of one expert form a bit-mask; the rank is the
//                    population count below the lane) plus the counts of earlier wavefronts, so
//                    dest_row[f] = offsets[e] + (earlier slots of e); sorted_src is its inverse
//   4. k_perm_rows   one wavefront per token reads its row once and writes it to its k
//                    destination rows (16-byte vectors): the row copy reads A exactly once
#include <mutex>

#include "common.h"

namespace fsm {

constexpr int PCH = 4096;  // slots per chunk (workgroup)
constexpr int PTHR = 256;

__global__ __launch_bounds__(PTHR) void k_perm_hist(const int32_t* __restrict__ idx, int64_t n, int E,
                                                    int32_t* __restrict__ counts) {
  __shared__ int32_t h[MOE_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += PTHR) h[e] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * PCH;
  for (int s = threadIdx.x; s < PCH; s += PTHR) {
    const int64_t f = base + s;
    if (f < n) atomicAdd(&h[idx[f]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PTHR) counts[int64_t(blockIdx.x) * E + e] = h[e];
}

// One block of 1024 threads; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ counts, int nblk, int E,
                                                    int32_t* __restrict__ base, int32_t* __restrict__ offsets) {
  __shared__ int32_t s[1024];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = 0; b < nblk; ++b) {
      const int c = counts[int64_t(b) * E + e];
      base[int64_t(b) * E + e] = run;
      run += c;
    }
  }
  s[e] = run;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (e >= off) ? s[e - off] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e] = s[e] - run;  // exclusive prefix
  if (e == 0) offsets[E] = s[1023];
}

__global__ __launch_bounds__(PTHR) void k_perm_rank(const int32_t* __restrict__ idx, int64_t n, int E,
                                                    int nbits, const int32_t* __restrict__ base,
                                                    const int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ sorted_src,
                                                    int32_t* __restrict__ dest_row) {
  __shared__ int32_t run[MOE_MAX_EXPERTS];
  __shared__ int32_t wc[PTHR / 64][MOE_MAX_EXPERTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += PTHR) {
    run[e] = offsets[e] + base[int64_t(blockIdx.x) * E + e];
#pragma unroll
    for (int w = 0; w < PTHR / 64; ++w) wc[w][e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  const int64_t chunk0 = int64_t(blockIdx.x) * PCH;
  for (int r0 = 0; r0 < PCH; r0 += PTHR) {
    const int64_t f = chunk0 + r0 + tid;
    const bool valid = f < n;
    const int e = valid ? idx[f] : E;  // E is a sentinel that matches no real expert
    uint64_t peers = ~uint64_t(0);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank_w = __popcll(peers & lt_mask);
    const int cnt_w = __popcll(peers);
    const bool leader = rank_w == 0;
    if (valid && leader) wc[wave][e] = cnt_w;
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += wc[w][e];
      const int r = run[e] + pre + rank_w;
      dest_row[f] = r;
      sorted_src[r] = int32_t(f);
    }
    __syncthreads();
    if (valid && leader) {
      atomicAdd(&run[e], cnt_w);
      wc[wave][e] = 0;
    }
    __syncthreads();
  }
}

// A_perm[dest_row[t*k+i]] = A[t]; row_vec = row length in 16-byte vectors.
typedef unsigned int pr_u32x4 __attribute__((ext_vector_type(4)));
constexpr int PR_UNROLL = 4;  // 16-byte vectors per lane in flight before the k stores

__global__ __launch_bounds__(256) void k_perm_rows(const pr_u32x4* __restrict__ A, int64_t T, int64_t row_vec,
                                                   int k, const int32_t* __restrict__ dest_row,
                                                   pr_u32x4* __restrict__ A_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myrow = lane < k ? dest_row[t * k + lane] : 0;
  const pr_u32x4* src = A + t * row_vec;
  // A is read once: nontemporal loads (plain stores measured 2% faster than nontemporal ones)
  for (int64_t c0 = lane; c0 < row_vec; c0 += 64 * PR_UNROLL) {
    pr_u32x4 v[PR_UNROLL];
#pragma unroll
    for (int u = 0; u < PR_UNROLL; ++u)
      if (c0 + 64 * u < row_vec) v[u] = __builtin_nontemporal_load(src + c0 + 64 * u);
    for (int i = 0; i < k; ++i) {
      pr_u32x4* dst = A_perm + int64_t(__builtin_amdgcn_readlane(myrow, i)) * row_vec + c0;
#pragma unroll
      for (int u = 0; u < PR_UNROLL; ++u)
        if (c0 + 64 * u < row_vec) dst[64 * u] = v[u];
    }
  }
}

size_t permute_ws_bytes(int64_t T, int32_t E, int32_t k) {
  const int64_t nblk = cdiv(T * k, PCH);
  return 2 * align_up(size_t(nblk) * size_t(E) * 4, 256) + 256;
}

int launch_permute(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                   const int32_t* topk_idx, int32_t* offsets, int32_t* sorted_src, int32_t* dest_row,
                   void* A_perm, void* ws, hipStream_t s) {
  const int64_t n = T * k;
  const int nblk = int(cdiv(n, PCH));
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                             align_up(size_t(nblk) * size_t(E) * 4, 256));
  {
    ProfScope prof(MOE_K_PERMUTE_INDEX, s);
    if (nblk > 0) {
      k_perm_hist<<<nblk, PTHR, 0, s>>>(topk_idx, n, E, counts);
      if (int rc = check_launch("permute histogram")) return rc;
    }
    k_perm_scan<<<1, 1024, 0, s>>>(counts, nblk, E, base, offsets);
    if (int rc = check_launch("permute scan")) return rc;
    if (nblk == 0) return MOE_OK;
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;  // enough bits for the values 0..E (E = sentinel)
    k_perm_rank<<<nblk, PTHR, 0, s>>>(topk_idx, n, E, nbits, base, offsets, sorted_src, dest_row);
    if (int rc = check_launch("permute rank")) return rc;
  }
  if (A_perm) {
    ProfScope prof(MOE_K_PERMUTE_ROWS, s);
    const int64_t row_bytes = d * (dtype == MOE_BF16 ? 2 : 4);
    k_perm_rows<<<unsigned(cdiv(T, 4)), 256, 0, s>>>(static_cast<const pr_u32x4*>(A), T, row_bytes / 16, k,
                                                    dest_row, static_cast<pr_u32x4*>(A_perm));
    if (int rc = check_launch("permute rows")) return rc;
  }
  return MOE_OK;
}

// ---- the permutation without a caller workspace (moe_permute_noalloc) ---------------------------
// The two per-chunk count arrays live in a fixed device array instead of a workspace argument.
// Every GPU the library runs on holds its own copy of the array until the process ends; host code
// reaches it only through the address that hipGetSymbolAddress returns for the current device (the
// array's name in host code is a host-side stand-in, not a device address).
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;   // MOE_PERMUTE_NOALLOC_SCRATCH_BYTES
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes == MOE_PERMUTE_NOALLOC_SCRATCH_BYTES, "header and library agree");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch` (looked up once per device, with that device current)
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_permute_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: device %d beyond the %d this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MOE_ERR_HIP, "moe_permute_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

size_t permute_noalloc_limit() { return kNoAllocScratchBytes; }

int launch_permute_noalloc(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                           const int32_t* topk_idx, int32_t* offsets, int32_t* sorted_src, int32_t* dest_row,
                           void* A_perm, hipStream_t s) {
  const size_t need = permute_ws_bytes(T, E, k);
  if (need > kNoAllocScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_permute_noalloc: T*k = %lld slots over E = %d experts need %zu bytes of scratch, above the "
                "fixed %zu (use moe_permute with a workspace)", (long long)(T * k), E, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  // k_perm_hist writes every count of every chunk and k_perm_scan every prefix before they are read,
  // so nothing in the scratch has to start at zero
  return launch_permute(A, dtype, T, d, E, k, topk_idx, offsets, sorted_src, dest_row, A_perm, ws, s);
}

}  // namespace fsm
