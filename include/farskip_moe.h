/*
 * farskip_moe.h -- C ABI of the MI355X (gfx950) MoE sublayer library, libfarskip_moe.so.
 *
 * One GPU's forward pass of a Mixture-of-Experts sublayer and of a FarSkip-Collective residual
 * stack built from such sublayers.  The operations follow the page "FarSkip-Collective:
 * Unhobbling Blocking Communication in Mixture of Experts Models" (papercache summary):
 *   section 2.1, modern MLP equation:  MLP(A) = sigma(A W1^T . g(A W2^T)) W3^T,
 *              W1, W2 in R^{c x d}, W3 in R^{d x c}; here g = SiLU, sigma = identity, '.' is
 *              the elementwise product;
 *   section 2.1, MoE equation:         MoE(A) = sum_j G(A)_j MLP^j(A), G(A) = s(A W_R^T);
 *   section 2.1, Dispatch / Combine:   token rows are permuted into expert-contiguous order, and
 *              the routed expert outputs are summed back per token;
 *   section 3, eqs. (8a)/(8b):         the FarSkip inputs o*_k ("outdated" / "partial").
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a DEVICE pointer to memory the caller owns (row-major, densely
 *     packed, 16-byte aligned), unless the argument says "host".  The library never allocates,
 *     frees or keeps device memory beyond the call, except that farskip_stack_forward creates
 *     HIP events that it destroys before returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).  All work is
 *     enqueued asynchronously on it; results are valid once the stream has been synchronised.
 *   - dtype: MOE_F32 (float32) or MOE_BF16 (bfloat16 storage, float32 accumulation).
 *   - Return value: MOE_OK (0) or a negative moe_status_t.  Argument checks run on the host
 *     before anything is enqueued; on an error nothing is enqueued and moe_last_error() returns a
 *     message (thread-local).  A failed kernel launch returns MOE_ERR_HIP.  Data-dependent
 *     preconditions (finite inputs, expert ids in [0, E), offsets non-decreasing) are the
 *     caller's and are not checked on the device.
 *   - No C++ exception crosses this interface.
 */
#ifndef FARSKIP_MOE_H
#define FARSKIP_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, k > E, inconsistent sizes */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, alignment, E or k too large) */
  MOE_ERR_WORKSPACE = -3,   /* workspace pointer null or ws_bytes below the queried size */
  MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;
typedef enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 } moe_gate_t;
typedef enum {
  FARSKIP_NONE = 0,     /* the standard residual stream (no skip) */
  FARSKIP_PARTIAL = 1,  /* MoE-only stack: next input o_{j-1} + shared output (eq. 8b) */
  FARSKIP_OUTDATED = 2, /* MoE-only stack: next input o_{j-1} (eq. 8a) */
  FARSKIP_PAPER = 3     /* attention + MoE stack: attention input partial, MoE input outdated */
} farskip_mode_t;

/* Limits of this implementation (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/*
 * moe_route -- router logits and top-k gating (section 2.1: G(A) = s(A W_R^T), a linear
 * classifier followed by a sparse selection s()).
 *
 *   A       [T, d] dtype      token activations
 *   W_R     [E, d] dtype      router weight (logits = A W_R^T)
 *   bias    [E] float32       optional per-expert logit bias (NULL = none)
 *   logits  [T, E] float32    OUTPUT logits = A W_R^T + bias.  If A and W_R are both NULL,
 *                             logits is instead an INPUT and only the selection runs (dtype,
 *                             d and bias are then ignored).
 *   topk_idx [T, k] int32     OUTPUT: per token the k experts with the largest logits, in
 *                             descending logit order; equal logits go to the lower expert index.
 *                             A NaN logit ranks below every number (it is taken as -infinity), so
 *                             every id is in [0, E) whatever the logits hold.
 *   topk_w  [T, k] float32    OUTPUT gate weights: gate = MOE_GATE_SOFTMAX -> softmax over all E
 *                             logits, evaluated at the selected experts; MOE_GATE_SIGMOID ->
 *                             1/(1+exp(-logit)).  renormalize != 0 divides by their sum over k.
 * Limits: 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS, bf16 needs d % 64 == 0.
 */
int moe_route(const void* A, const void* W_R, const float* bias, int dtype, int64_t T, int64_t d,
              int32_t E, int32_t k, int gate, int renormalize, float* logits, int32_t* topk_idx,
              float* topk_w, void* stream);

/*
 * moe_permute -- the Dispatch permutation of section 2.1 on one GPU: every (token t, slot i)
 * pair becomes one row; rows are grouped by expert, and inside an expert ordered by the flat
 * slot f = t*k + i (a stable counting sort).
 *
 *   topk_idx       [T, k] int32   expert of each slot (values in [0, E))
 *   expert_offsets [E+1] int32    OUTPUT: rows of expert e are [offsets[e], offsets[e+1])
 *   sorted_src     [T*k] int32    OUTPUT: flat slot placed at each row
 *   dest_row       [T*k] int32    OUTPUT: row of each flat slot (inverse of sorted_src)
 *   A              [T, d] dtype   token activations, may be NULL when A_perm is NULL
 *   A_perm         [T*k, d] dtype OUTPUT (optional, NULL = skip): A_perm[dest_row[t*k+i]] = A[t]
 *   ws, ws_bytes   scratch of at least moe_permute_workspace_bytes(T, E, k) bytes
 * All outputs are deterministic (bit-identical from run to run).
 */
int moe_permute(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_src,
                int32_t* dest_row, void* A_perm, void* ws, size_t ws_bytes, void* stream);
size_t moe_permute_workspace_bytes(int64_t T, int32_t E, int32_t k);

/*
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device memory or pass a
 * workspace: code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation.  Same arguments and outputs as moe_permute, bit for bit, without ws / ws_bytes: the
 * scratch (the per-chunk expert counts and their prefix sums, moe_permute_workspace_bytes(T, E, k)
 * bytes) lives in a fixed device array of MOE_PERMUTE_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, held until the process ends.  The call allocates and frees nothing; its first call on a
 * device looks up that device's array (the current device must be the stream's device).
 * Sizes whose scratch exceeds the array (roughly T * k * E > 4096 * 2^20) return MOE_ERR_UNSUPPORTED
 * with a message; other errors as moe_permute.  Nothing in the array has to start at zero.  All calls
 * on one GPU share its array: two such calls that may run at the same time on that GPU (on
 * different streams, or from different host threads) race and must be ordered by the caller.
 */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int moe_permute_noalloc(const void* A, int dtype, int64_t T, int64_t d, int32_t E, int32_t k,
                        const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_src,
                        int32_t* dest_row, void* A_perm, void* stream);

/*
 * moe_grouped_swiglu -- the modern MLP of section 2.1 applied per group (expert):
 * for rows r in [group_offsets[g], group_offsets[g+1]):
 *     H[r] = (X[r] W1[g]^T) . SiLU(X[r] W2[g]^T)      (H kept in dtype, in the workspace)
 *     Y[r] = H[r] W3[g]^T
 *
 *   X             [N, d] dtype     input rows, grouped (e.g. A_perm from moe_permute)
 *   group_offsets [G+1] int32      device array, non-decreasing, offsets[0] = 0, offsets[G] = N
 *   W1, W2        [G, c, d] dtype  up and gate projections (row-major c x d per group)
 *   W3            [G, d, c] dtype  down projection (row-major d x c per group)
 *   Y             [N, d] dtype     OUTPUT
 *   ws, ws_bytes  scratch of at least moe_grouped_swiglu_workspace_bytes(N, G, c, dtype)
 * A shared expert is the call with G = 1 and offsets {0, T}; several shared experts are one call
 * with their hidden dimensions concatenated (c = n_shared * c_shared).
 * Limits: bf16 needs d % 64 == 0 and c % 64 == 0.
 */
int moe_grouped_swiglu(const void* X, const int32_t* group_offsets, int32_t G, const void* W1,
                       const void* W2, const void* W3, int dtype, int64_t N, int64_t d, int64_t c,
                       void* Y, void* ws, size_t ws_bytes, void* stream);
size_t moe_grouped_swiglu_workspace_bytes(int64_t N, int32_t G, int64_t c, int dtype);

/*
 * moe_grouped_swiglu_gathered -- moe_grouped_swiglu with the Dispatch permutation of section 2.1
 * folded into its loads: grouped row r is token row X[sorted_src[r] / k], so the permuted copy
 * of the activations (A_perm) is never written.  Same result, bit for bit, as moe_permute with
 * A_perm followed by moe_grouped_swiglu on A_perm.
 *
 *   X             [T, d] dtype    token activations
 *   sorted_src    [N] int32       flat slot of each grouped row (moe_permute output); values in [0, T*k)
 *   k             slots per token (sorted_src[r] / k is the token)
 *   other arguments as moe_grouped_swiglu (N rows, G groups, workspace of the same size)
 * Limits: as moe_grouped_swiglu; bf16 also needs T * d * 2 < 2^31 bytes.
 */
int moe_grouped_swiglu_gathered(const void* X, int64_t T, const int32_t* sorted_src, int32_t k,
                                const int32_t* group_offsets, int32_t G, const void* W1, const void* W2,
                                const void* W3, int dtype, int64_t N, int64_t d, int64_t c, void* Y,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * MXFP8 expert products.  FarSkip-Collective's inference measurements run the MoE forward with FP8
 * quantisation (the page's experimental setup: software configuration and inference parameters);
 * the pages name no format.  Format taken: OCP MXFP8 -- FP8 E4M3 elements (largest magnitude 448,
 * subnormals kept, nearest value with ties to the even code) and one E8M0 power-of-two scale per
 * 32 consecutive elements along the reduction dimension.  Block scale: the smallest 2^s with
 * max|x| / 2^s <= 448 (0 for an all-zero block), stored as the byte s + 127.
 *
 * moe_mx_quantize -- rows of bf16 X to MXFP8.
 *   X       [rows, K] bf16      input (device)
 *   codes   [rows, K] uint8     OUTPUT E4M3 codes, row-major
 *   scales  [rows, K/32] uint8  OUTPUT E8M0 scales; byte j of a row covers its elements 32j .. 32j+31
 * Weights are quantised by the same call (W1 / W2 as [G*c, d] along d, W3 as [G*d, c] along c).
 * Limits: K % 32 == 0; non-finite inputs are not supported.
 */
int moe_mx_quantize(const void* X, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * moe_grouped_swiglu_mxfp8 -- moe_grouped_swiglu with MXFP8 operands (all pointers device):
 *     H[r] = (X[r] W1[g]^T) . SiLU(X[r] W2[g]^T)   fp32 accumulation of the dequantised products,
 *                                                   H formed in fp32 and quantised to MXFP8 along c
 *     Y[r] = H[r] W3[g]^T                           fp32 accumulation, Y stored as bf16
 *
 *   Xq, Xs        [x_rows, d] / [x_rows, d/32] uint8   activation codes and scales (moe_mx_quantize)
 *   x_rows        rows of Xq (N when sorted_src is NULL; the token count T when gathering)
 *   sorted_src    NULL: grouped row r is Xq row r.  Else [N] int32 (moe_permute output, values in
 *                 [0, x_rows * k)): grouped row r is Xq row sorted_src[r] / k -- the Dispatch
 *                 permutation of section 2.1 folded into the loads; the result is bit-identical
 *   k             slots per token (used only with sorted_src)
 *   group_offsets [G+1] int32      as moe_grouped_swiglu
 *   W1q, W1s      [G, c, d] / [G, c, d/32] uint8   up projection, quantised along d
 *   W2q, W2s      [G, c, d] / [G, c, d/32] uint8   gate projection, quantised along d
 *   W3q, W3s      [G, d, c] / [G, d, c/32] uint8   down projection, quantised along c
 *   Y             [N, d] bf16      OUTPUT, grouped row order
 *   ws, ws_bytes  scratch of at least moe_grouped_swiglu_mxfp8_workspace_bytes(N, G, c); after the
 *                 call it holds H's codes and scales (not part of the interface)
 * Limits: d % 128 == 0, c % 128 == 0, x_rows * d < 2^31.
 */
int moe_grouped_swiglu_mxfp8(const uint8_t* Xq, const uint8_t* Xs, int64_t x_rows, const int32_t* sorted_src,
                             int32_t k, const int32_t* group_offsets, int32_t G, const uint8_t* W1q,
                             const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s, const uint8_t* W3q,
                             const uint8_t* W3s, int64_t N, int64_t d, int64_t c, void* Y, void* ws,
                             size_t ws_bytes, void* stream);
size_t moe_grouped_swiglu_mxfp8_workspace_bytes(int64_t N, int32_t G, int64_t c);

/*
 * The two products of moe_grouped_swiglu_mxfp8 as calls of their own (H in the caller's buffers);
 * gate_up followed by down gives the fused call's Y bit for bit.
 *
 * moe_grouped_mxfp8_gate_up -- H = (X W1^T) . SiLU(X W2^T), formed in fp32, quantised along c.
 *   Xq .. W2s, N, d, c     as moe_grouped_swiglu_mxfp8
 *   Hq, Hs                 [N, c] / [N, c/32] uint8   OUTPUT H codes and scales, grouped row order
 * moe_grouped_mxfp8_down -- Y = H W3^T per group, fp32 accumulation, Y stored as bf16.
 *   Hq, Hs                 [N, c] / [N, c/32] uint8   (e.g. moe_grouped_mxfp8_gate_up output)
 *   W3q, W3s, Y, N, c, d   as moe_grouped_swiglu_mxfp8 (note the argument order c, d)
 * Both: ws of at least moe_grouped_mxfp8_phase_workspace_bytes(N, G) bytes (the group tile
 * table); same limits as moe_grouped_swiglu_mxfp8.
 */
int moe_grouped_mxfp8_gate_up(const uint8_t* Xq, const uint8_t* Xs, int64_t x_rows, const int32_t* sorted_src,
                              int32_t k, const int32_t* group_offsets, int32_t G, const uint8_t* W1q,
                              const uint8_t* W1s, const uint8_t* W2q, const uint8_t* W2s, int64_t N, int64_t d,
                              int64_t c, uint8_t* Hq, uint8_t* Hs, void* ws, size_t ws_bytes, void* stream);
int moe_grouped_mxfp8_down(const uint8_t* Hq, const uint8_t* Hs, const int32_t* group_offsets, int32_t G,
                           const uint8_t* W3q, const uint8_t* W3s, int64_t N, int64_t c, int64_t d, void* Y,
                           void* ws, size_t ws_bytes, void* stream);
size_t moe_grouped_mxfp8_phase_workspace_bytes(int64_t N, int32_t G);

/*
 * moe_combine -- the Combine of section 2.1: routed expert outputs summed back per token.
 *   out[t] = residual[t] + addend[t] + sum_{i<k} topk_w[t,i] * Y[dest_row[t*k+i]]
 * accumulated in float32, slots in order i = 0..k-1 (deterministic, no atomics).
 *
 *   Y        [T*k, d] dtype   expert outputs in permuted row order
 *   topk_w   [T, k] float32   gate weights
 *   dest_row [T*k] int32      row of each flat slot (from moe_permute)
 *   addend   [T, d] dtype     optional (NULL = 0), e.g. the shared-expert output
 *   residual [T, d] float32   optional (NULL = 0), e.g. the residual stream o_{k-1}
 *   out      [T, d] float32   OUTPUT; may alias residual (in-place update of the stream)
 *   out_x    [T, d] dtype     optional OUTPUT: out rounded to dtype (next layer's input)
 */
int moe_combine(const void* Y, int dtype, const float* topk_w, const int32_t* dest_row, int64_t T,
                int64_t d, int32_t k, const void* addend, const float* residual, float* out,
                void* out_x, void* stream);

/* One MoE sublayer's weights for farskip_stack_forward (device pointers, layouts as above). */
typedef struct {
  const void* W_R;   /* [E, d] */
  const float* bias; /* [E] or NULL */
  const void* W1;    /* [E, c, d] */
  const void* W2;    /* [E, c, d] */
  const void* W3;    /* [E, d, c] */
  const void* Ws1;   /* [c_shared, d] or NULL when c_shared == 0 */
  const void* Ws2;   /* [c_shared, d] */
  const void* Ws3;   /* [d, c_shared] */
} moe_layer_desc_t;

/* Shapes and gating shared by every layer of a stack. */
typedef struct {
  int64_t T, d, c;   /* tokens, model width, routed expert hidden width */
  int64_t c_shared;  /* total shared hidden width (n_shared * per-expert width), 0 = none */
  int32_t E, k;      /* routed experts, experts per token */
  int32_t gate;      /* moe_gate_t */
  int32_t renormalize;
  int32_t dtype;     /* moe_dtype_t of activations and weights */
} moe_stack_cfg_t;

/*
 * Timing of one stack call, measured on the device with events around each of its kernels (the
 * analogue of the share of communication hidden behind computation that section 4 of the page
 * reports: here the second queue's kernel time that runs while the first queue's does).  Times are
 * milliseconds; M is the union of s_main's kernel intervals and S that of s_side's.
 */
typedef struct {
  double wall_ms;          /* first kernel start to last kernel end, both streams */
  double main_busy_ms;     /* |M| */
  double side_busy_ms;     /* |S| */
  double overlap_ms;       /* |M intersect S| */
  double overlap_of_side;  /* |M intersect S| / |S| (0 when S is empty) */
  double overlap_of_main;  /* |M intersect S| / |M| (0 when M is empty) */
  int32_t launches_main;   /* kernels on s_main */
  int32_t launches_side;   /* kernels on s_side (0 when s_side == s_main) */
} moe_stack_stats_t;

/*
 * farskip_stack_forward -- L MoE sublayers f_j = S_j + R_j (shared + routed) on the residual
 * stream, wired as section 3 of the page describes:
 *     o_j = o_{j-1} + S_j(x_j) + R_j(x_j),  x_1 = o_0, and
 *     x_{j+1} = o_j                      if mode == FARSKIP_NONE or skip_mask[j] == 0,
 *     x_{j+1} = o_{j-1} + S_j(x_j)       if mode == FARSKIP_PARTIAL  (eq. 8b, f* = shared expert),
 *     x_{j+1} = o_{j-1}                  if mode == FARSKIP_OUTDATED (eq. 8a).
 * The residual o_j is kept in float32; each layer input x_j is rounded to cfg->dtype.
 * s_main runs each layer's permutation and routed grouped GEMM (rows gathered through the
 * permutation), and nothing else.  s_side runs each layer's router and shared expert, the
 * previous layer's combine and, with the skip on, the next layer's input; with the skip on at
 * layer j, layer j's shared expert, layer j-1's combine (which also forms x_{j+1}) and layer
 * j+1's router all run while layer j's routed GEMMs do: they wait until layer j's routed gate/up
 * product is done and run beside its down product (HIP events order the two streams).
 * s_side == s_main gives the same results with everything serialised on one stream.  Inputs
 * are taken as ordered on s_main: s_side first waits for all work enqueued on s_main before the
 * call, and s_main's last operation waits for the final combine, so the result is ready when
 * s_main is.  The call allocates no device memory, does not synchronise with the host and issues
 * no memset, so it may be captured into a HIP graph on s_main (s_side then joins the capture
 * through the call's first event wait); each replay recomputes o_L from the current contents of
 * o0, the weights and the workspace pointers given at capture.
 *
 *   layers    host array [L] of device-pointer descriptors
 *   cfg       host pointer
 *   skip_mask host array [L] of 0/1, or NULL = skip on for every layer
 *   o0        [T, d] float32 input o_0;  oL [T, d] float32 OUTPUT o_L (must not alias o0)
 *   ws        scratch of at least farskip_stack_workspace_bytes(cfg) bytes
 *   stats     host pointer or NULL.  NULL: the call is asynchronous, as described above.  Non-NULL:
 *             every kernel of this call is bracketed by timing events on its own stream, the call
 *             waits until s_main (and so the whole stack) has finished, and fills *stats (see
 *             moe_stack_stats_t).  Those launches are not seen by moe_profile_collect.  A non-NULL
 *             stats while s_main is being captured into a graph returns MOE_ERR_INVALID_ARG.
 */
int farskip_stack_forward(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t* cfg,
                          int mode, const uint8_t* skip_mask, const float* o0, float* oL, void* ws,
                          size_t ws_bytes, void* s_main, void* s_side, moe_stack_stats_t* stats);
size_t farskip_stack_workspace_bytes(const moe_stack_cfg_t* cfg);

/* The weights of the dense SwiGLU block that stands in for a layer's attention sub-block in
 * farskip_attn_moe_stack_forward (device pointers): Wa1, Wa2 [c_attn, d], Wa3 [d, c_attn]. */
typedef struct {
  const void* Wa1;
  const void* Wa2;
  const void* Wa3;
} moe_attn_desc_t;

/*
 * farskip_attn_moe_stack_forward -- L layers, each an attention sub-block followed by an MoE
 * sub-block (shared experts S_j plus routed experts R_j), on the residual stream, wired as section 3
 * of the page gives it for such models:
 *   mode FARSKIP_PAPER: the attention input is the partial activation (eq. 8b) and the MoE input the
 *       outdated one (eq. 8a):
 *         attn-in_j = o_{j-2} + attn-out_{j-1} + S_{j-1}   (everything in o_{j-1} but R_{j-1}; o_0 at j = 1)
 *         mlp-in_j  = o_{j-1} = attn-in_j + R_{j-1}
 *   mode FARSKIP_NONE: the standard stream, attn-in_j = o_{j-1}, mlp-in_j = o_{j-1} + attn-out_j;
 *   in both: o_j = o_{j-1} + attn-out_j + S_j(mlp-in_j) + R_j(mlp-in_j).
 * No attention block is in this library: each attention sub-block is computed by a dense SwiGLU
 * block of hidden width c_attn with the layer's attn[j] weights (the wiring does not depend on what
 * the sub-block computes).  The residual is float32; every sub-block input is rounded to
 * cfg->dtype.  Streams: s_main runs each layer's permutation and routed GEMMs; s_side runs the
 * routers, shared experts, combines and attention blocks -- in FARSKIP_PAPER mode layer j+1's
 * attention runs while layer j's routed experts do.  s_side == s_main serialises everything with the
 * same results.  Stream contract, graph capture and stats as farskip_stack_forward.
 *   layers, L, cfg, o0, oL   as farskip_stack_forward
 *   attn     host array [L] of the attention stand-ins' weights
 *   c_attn   their hidden width (bf16: a multiple of 64)
 *   ws       scratch of at least farskip_attn_moe_stack_workspace_bytes(cfg, c_attn) bytes
 */
int farskip_attn_moe_stack_forward(const moe_layer_desc_t* layers, const moe_attn_desc_t* attn, int32_t L,
                                   const moe_stack_cfg_t* cfg, int64_t c_attn, int mode, const float* o0,
                                   float* oL, void* ws, size_t ws_bytes, void* s_main, void* s_side,
                                   moe_stack_stats_t* stats);
size_t farskip_attn_moe_stack_workspace_bytes(const moe_stack_cfg_t* cfg, int64_t c_attn);

/* MXFP8 codes and scales of one layer's expert weights, as moe_mx_quantize writes them. */
typedef struct {
  const uint8_t* W1q;  /* [E, c, d] E4M3 codes */
  const uint8_t* W1s;  /* [E, c, d / 32] E8M0 scales */
  const uint8_t* W2q;  /* [E, c, d] */
  const uint8_t* W2s;  /* [E, c, d / 32] */
  const uint8_t* W3q;  /* [E, d, c] */
  const uint8_t* W3s;  /* [E, d, c / 32] */
  const uint8_t* Ws1q; /* [c_shared, d] shared experts (NULL when c_shared == 0) */
  const uint8_t* Ws1s; /* [c_shared, d / 32] */
  const uint8_t* Ws2q; /* [c_shared, d] */
  const uint8_t* Ws2s; /* [c_shared, d / 32] */
  const uint8_t* Ws3q; /* [d, c_shared] */
  const uint8_t* Ws3s; /* [d, c_shared / 32] */
} moe_layer_mx_t;

/*
 * farskip_stack_forward_mxfp8 -- farskip_stack_forward with each layer's expert MLPs (routed and
 * shared) run on MXFP8 operands (FarSkip-Collective section 5 serves its converted models with FP8
 * quantisation and fused MoE kernels; the format is OCP MXFP8).  Per layer, on top of the bf16
 * stack: the layer input x_j (bf16) is quantised to MXFP8 rows on s_side right after it is formed;
 * s_main's routed products are moe_grouped_swiglu_mxfp8 with rows gathered through the permutation
 * and s_side's shared expert is moe_grouped_swiglu_mxfp8 over all T rows as one group (outputs in
 * bf16).  The router, top-k, combine and the residual bookkeeping are those of
 * farskip_stack_forward, in bf16 / fp32.  The result equals the same single calls composed on one
 * stream, bit for bit.  Streams, events and graph capture as for farskip_stack_forward.
 *   layers  as farskip_stack_forward, except that W1-W3 and Ws1-Ws3 are not read (may be NULL)
 *   mx      host array [L]: the experts' MXFP8 codes and scales
 *   ws      scratch of at least farskip_stack_mxfp8_workspace_bytes(cfg) bytes
 * Requires cfg->dtype == MOE_BF16, d, c and c_shared multiples of 128.  Errors, stream contract and
 * stats as farskip_stack_forward.
 */
int farskip_stack_forward_mxfp8(const moe_layer_desc_t* layers, const moe_layer_mx_t* mx, int32_t L,
                                const moe_stack_cfg_t* cfg, int mode, const uint8_t* skip_mask, const float* o0,
                                float* oL, void* ws, size_t ws_bytes, void* s_main, void* s_side,
                                moe_stack_stats_t* stats);
size_t farskip_stack_mxfp8_workspace_bytes(const moe_stack_cfg_t* cfg);

/*
 * moe_layer_backward -- the backward pass of one MoE sublayer: the gradients of its output
 * out = S(A) + R(A) (section 2.1: router G(A) = s(A W_R^T) + b, the modern MLP per expert,
 * Dispatch, Combine with the gate weights, and the shared experts S) with respect to the input A
 * and every weight, given dOut = dLoss/dout.  The chain rule of the forward, in reverse; the top-k
 * choice itself passes no gradient (only the selected experts' weights do).  The page's training
 * schedule (section 4.1) runs this pass for every MoE layer; this call is one GPU's share.
 *
 *   W            host pointer: the layer's weights (as for farskip_stack_forward)
 *   cfg          host pointer: T, d, c, c_shared, E, k, gate, renormalize; dtype must be MOE_BF16
 *   A            [T, d] bf16        the layer input of the forward
 *   logits       [T, E] float32     the forward's router logits (bias included)
 *   topk_idx, topk_w                the forward's selection and gate weights ([T, k])
 *   expert_offsets, sorted_src, dest_row   the forward's permutation (moe_permute)
 *   Y            [T*k, d] bf16      the forward's routed expert outputs (grouped row order)
 *   dOut         [T, d] float32     gradient of the loss with respect to out
 *   dOut_shared  [T, d] float32 or NULL: the shared experts' own output gradient when it differs
 *                from dOut (in a FarSkip stack the shared output also feeds the next layer's
 *                input, eq. 8b); NULL = dOut
 *   grads        host pointer to OUTPUT device pointers, all float32, overwritten:
 *                  dA [T, d] (the residual's own pass-through is not included), dW_R [E, d],
 *                  dbias [E] (or NULL: not computed), dW1, dW2 [E, c, d], dW3 [E, d, c], and
 *                  with c_shared > 0 dWs1, dWs2 [c_shared, d], dWs3 [d, c_shared]
 *   ws, ws_bytes scratch of at least moe_layer_backward_workspace_bytes(cfg) bytes
 * Intermediates (dY, the recomputed U and G, H, dH, dU, dG, dX and the router's dlogits) are kept
 * in bf16 and every product accumulates in fp32.
 * Limits: bf16 only; d, c and c_shared multiples of 64; E a multiple of 8; T * d * 2 < 2^31.
 */
typedef struct {
  float* dA;
  float* dW_R;
  float* dbias;
  float* dW1;
  float* dW2;
  float* dW3;
  float* dWs1;
  float* dWs2;
  float* dWs3;
} moe_layer_grads_t;

int moe_layer_backward(const moe_layer_desc_t* W, const moe_stack_cfg_t* cfg, const void* A, const float* logits,
                       const int32_t* topk_idx, const float* topk_w, const int32_t* expert_offsets,
                       const int32_t* sorted_src, const int32_t* dest_row, const void* Y, const float* dOut,
                       const float* dOut_shared, const moe_layer_grads_t* grads, void* ws, size_t ws_bytes,
                       void* stream);
size_t moe_layer_backward_workspace_bytes(const moe_stack_cfg_t* cfg);

/*
 * farskip_stack_backward -- the backward pass of the FarSkip stack of farskip_stack_forward
 * (section 3, eqs. (8a)/(8b)) for dOL = dLoss/do_L: dO0 = dLoss/do_0 and every layer's weight
 * gradients.  The forward is replayed on the stream keeping each layer's input, routing and expert
 * outputs; then the layers' backward passes (moe_layer_backward) run from the last layer to the
 * first with the gradients routed along the stack's graph: o_j feeds o_{j+1} and the next input
 * (x_{j+1} = o_j without the skip, x_{j+2} = o_j (+ S_{j+1}) with it), and under "partial" the
 * shared output S_j also feeds x_{j+1}, so the shared experts of layer j receive
 * dLoss/do_j + dLoss/dx_{j+1} while the routed ones receive dLoss/do_j.  The rounding of the layer
 * inputs to bf16 passes gradients through unchanged.  One stream; bf16 only.
 *
 *   layers, L, cfg, mode, skip_mask, o0   as for farskip_stack_forward
 *   dOL    [T, d] float32   gradient of the loss with respect to o_L
 *   dO0    [T, d] float32   OUTPUT gradient with respect to o_0 (must not alias dOL)
 *   grads  host array [L]: each layer's gradient outputs as for moe_layer_backward; dA (optional)
 *          receives dLoss/dx_j, the gradient with respect to that layer's input
 *   ws     scratch of at least farskip_stack_backward_workspace_bytes(cfg, L) bytes
 * Limits: as moe_layer_backward.
 */
int farskip_stack_backward(const moe_layer_desc_t* layers, int32_t L, const moe_stack_cfg_t* cfg, int mode,
                           const uint8_t* skip_mask, const float* o0, const float* dOL, float* dO0,
                           const moe_layer_grads_t* grads, void* ws, size_t ws_bytes, void* stream);
size_t farskip_stack_backward_workspace_bytes(const moe_stack_cfg_t* cfg, int32_t L);

/*
 * moe_workspace_bytes -- the scratch size of the MoE entry points, as one call: a dispatch over the
 * per-call queries above (farskip_attn_moe_stack_forward, which also needs the attention width, has
 * its own query).  The sizes are those of one MoE layer (section 2.1: T tokens of width d,
 * E routed experts of hidden width c, k experts per token, shared experts of total hidden width
 * c_shared) and of an L-layer stack:
 *   MOE_OP_PERMUTE                moe_permute for T tokens, E experts, k slots
 *   MOE_OP_GROUPED_SWIGLU         moe_grouped_swiglu(_gathered) over the layer's routed rows:
 *                                 N = T * k rows in G = E groups of hidden width c, dtype
 *                                 (the shared expert: E = 1, k = 1, c = c_shared)
 *   MOE_OP_GROUPED_SWIGLU_MXFP8   moe_grouped_swiglu_mxfp8, same N, G, c
 *   MOE_OP_MXFP8_PHASE            moe_grouped_mxfp8_gate_up / _down, same N, G
 *   MOE_OP_STACK                  farskip_stack_forward (L is not needed: buffers are reused)
 *   MOE_OP_STACK_MXFP8            farskip_stack_forward_mxfp8
 *   MOE_OP_LAYER_BACKWARD         moe_layer_backward
 *   MOE_OP_STACK_BACKWARD         farskip_stack_backward with L layers
 * The first seven arguments follow the order (op, T, d, E, k, c, L); c_shared and dtype (a
 * moe_dtype_t) complete the layer description.  The gate does not change any size.  Returns 0 for
 * an unknown op or sizes the op rejects (as the per-call queries do).
 */
typedef enum {
  MOE_OP_PERMUTE = 0,
  MOE_OP_GROUPED_SWIGLU = 1,
  MOE_OP_GROUPED_SWIGLU_MXFP8 = 2,
  MOE_OP_MXFP8_PHASE = 3,
  MOE_OP_STACK = 4,
  MOE_OP_STACK_MXFP8 = 5,
  MOE_OP_LAYER_BACKWARD = 6,
  MOE_OP_STACK_BACKWARD = 7
} moe_op_t;

size_t moe_workspace_bytes(int op, int64_t T, int64_t d, int32_t E, int32_t k, int64_t c, int32_t L,
                           int64_t c_shared, int dtype);

/*
 * Kernel timing for measurement harnesses.  While enabled (process-wide), every kernel the
 * library launches is bracketed by two timing hipEvents recorded on the stream it is launched on.
 * moe_profile_collect waits for the recorded events, returns per-kind launch counts and summed
 * durations (milliseconds), and clears the records.  Kinds are the moe_kernel_kind_t values; out
 * must hold MOE_KERNEL_KINDS entries.  Disabled by default; enabling costs two event records per
 * launch.
 */
typedef enum {
  MOE_K_ROUTER_GEMM = 0,  /* logits = A W_R^T */
  MOE_K_TOPK = 1,         /* top-k selection and gate weights */
  MOE_K_PERMUTE_INDEX = 2,/* histogram + scan + stable rank (all three kernels) */
  MOE_K_PERMUTE_ROWS = 3, /* A -> A_perm row copy */
  MOE_K_TILE_TABLE = 4,   /* grouped GEMM M-tile table */
  MOE_K_GEMM_GATE_UP = 5, /* grouped GEMM phase 1, G > 1: H = (X W1^T) . SiLU(X W2^T) */
  MOE_K_GEMM_DOWN = 6,    /* grouped GEMM phase 2, G > 1: Y = H W3^T */
  MOE_K_COMBINE = 7,      /* combine */
  MOE_K_LAYER_INPUT = 8,  /* FarSkip layer input x = cast(o [+ S]) */
  MOE_K_DENSE_GATE_UP = 9,/* phase 1 of a single-group call (e.g. the shared expert) */
  MOE_K_DENSE_DOWN = 10,  /* phase 2 of a single-group call */
  MOE_K_MX_QUANTIZE = 11, /* MXFP8 quantisation of rows */
  MOE_K_MX_GATE_UP = 12,  /* MXFP8 grouped product, phase 1 (with H quantised in its epilogue) */
  MOE_K_MX_DOWN = 13,     /* MXFP8 grouped product, phase 2 */
  MOE_K_BWD_RECOMPUTE = 14, /* backward: U and G recomputed (routed and shared) */
  MOE_K_BWD_DGRAD = 15,   /* backward: products giving activation gradients (dH, dX, router dA) */
  MOE_K_BWD_WGRAD = 16,   /* backward: weight-gradient products (reduction over rows) */
  MOE_K_TRANSPOSE = 17,   /* backward: weight and activation transposes */
  MOE_K_BWD_POINTWISE = 18, /* backward: combine, gate, SwiGLU and bias-sum kernels */
  MOE_K_MX_DENSE_GATE_UP = 19, /* MXFP8 phase 1 of a single-group call (the shared expert) */
  MOE_K_MX_DENSE_DOWN = 20,    /* MXFP8 phase 2 of a single-group call */
  MOE_K_ATTN_GATE_UP = 21,     /* attention stand-in block (farskip_attn_moe_stack_forward), phase 1 */
  MOE_K_ATTN_DOWN = 22,        /* attention stand-in block, phase 2 */
  MOE_KERNEL_KINDS = 23
} moe_kernel_kind_t;

typedef struct {
  int32_t count;   /* launches recorded */
  double total_ms; /* summed event-to-event durations */
} moe_kernel_time_t;

int moe_profile_enable(int on);
int moe_profile_collect(moe_kernel_time_t* out /* [MOE_KERNEL_KINDS] */);

/*
 * One recorded launch on a common time axis, for the cross-stream overlap of the FarSkip stack
 * (the share of the second queue's work that runs while the first queue's runs).
 */
typedef struct {
  int32_t kind;     /* moe_kernel_kind_t */
  int32_t pad;
  uint64_t stream;  /* the hipStream_t it was launched on, as an opaque id */
  double start_ms;  /* start event, ms relative to the first recorded launch's start event (negative
                       for a launch on another stream that started before it) */
  double end_ms;    /* end event, same origin */
} moe_kernel_interval_t;

/*
 * moe_profile_collect, plus each recorded launch's interval in record order.
 *   out       [MOE_KERNEL_KINDS] per-kind totals, as moe_profile_collect
 *   iv        host array of cap entries; the first min(cap, launches) launches are written
 *   n         receives the number of recorded launches (may exceed cap)
 * Clears the records.  Errors: out, iv (with cap > 0) or n null -> MOE_ERR_INVALID_ARG; a failed
 * event query -> MOE_ERR_HIP (records are still released).
 */
int moe_profile_collect_intervals(moe_kernel_time_t* out, moe_kernel_interval_t* iv, int32_t cap, int32_t* n);

/*
 * Diagnostic, not part of the method: the chip's register-only bf16 MFMA throughput, the ceiling
 * the products' MFMA fractions can be read against (the published dense peak assumes a clock the
 * chip does not hold under a full matrix load).  Launches `blocks` workgroups of 512 threads on
 * `stream`; each of their waves runs `iters` rounds of 16 independent MFMAs on register operands
 * with no memory traffic, and writes one float per thread to out.
 *   shape   0: v_mfma_f32_16x16x32_bf16 (the instruction the bf16 products use), 262 144 FLOP per
 *              wave and round;
 *           1: v_mfma_f32_32x32x16_bf16 (8 accumulators), 262 144 FLOP per wave and round;
 *           2: v_mfma_scale_f32_16x16x128_f8f6f4 on E4M3 codes (the MXFP8 products' instruction),
 *              1 048 576 FLOP per wave and round
 *   out     device buffer of blocks * 512 floats (caller-owned; values meaningless)
 * FLOP of one launch = blocks * 8 * iters * (FLOP per wave and round); time it with events on
 * `stream`.  Errors: shape not 0/1/2, iters < 1, blocks < 1 or out null -> MOE_ERR_INVALID_ARG;
 * launch -> MOE_ERR_HIP.
 */
int moe_mfma_ceiling(int shape, int32_t iters, int32_t blocks, float* out, void* stream);

/*
 * Diagnostic, not part of the method: how fast a product's operand stream can reach LDS, the
 * ceiling its K steps can be read against once the L2 hit rate is known.  Launches `blocks`
 * workgroups of 512 threads on `stream` (each takes 128 KB of LDS, so one runs per CU); each runs
 * `iters` stages of 64 KiB, loaded as a bf16 product's K step loads its two operand tiles: 64 runs
 * of 1 KiB per stage, one 16-byte direct-to-LDS load per lane, then a wait and a barrier; no
 * arithmetic.  Run r of stage i reads the hot window (the buffer's first MiB, which stays in
 * every XCD's L2) when (7 r + 3 i) mod 100 < hot_pct, else the workgroup's own cold region
 * (cold_bytes at offset 16 MiB + block * cold_bytes, swept in order: beyond the memory-side cache
 * when blocks * cold_bytes is large, inside it when small).  Exactly hot_pct of every 100 stages'
 * runs are hot.
 *   in_flight  1: a stage is requested once the previous one has landed (the two-stage ring of the
 *              products: one stage loads while the other is read); 2: two stages in flight
 *   buf        device buffer of buf_bytes >= 16 MiB + blocks * cold_bytes (caller-owned; only read)
 *   out        device buffer of blocks * 512 floats: each thread's sum of one byte of each LDS stage
 *   clocks     device buffer of 2 uint64 or NULL: workgroup 0's loop in shader-clock cycles
 *              (s_memtime) and in ticks of the 100 MHz constant counter (s_memrealtime), so
 *              clocks[0] / clocks[1] * 0.1 is the shader clock in GHz the probe ran at
 * Bytes of one launch = blocks * iters * 65536; time it with events on `stream`.  Errors: hot_pct
 * outside [0, 100], cold_bytes not a positive multiple of 128, iters < 1, blocks < 1, in_flight
 * not 1/2, buf or out null, or buf_bytes too small -> MOE_ERR_INVALID_ARG; 16 MiB + blocks *
 * cold_bytes >= 2 GiB -> MOE_ERR_UNSUPPORTED; launch -> MOE_ERR_HIP.
 */
int moe_delivery_probe(int32_t hot_pct, int64_t cold_bytes, int32_t iters, int32_t in_flight, int32_t blocks,
                       const void* buf, int64_t buf_bytes, float* out, uint64_t* clocks, void* stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FARSKIP_MOE_H */
