/*
 * moe_mi355x.h -- C ABI of the routed Mixture-of-Experts FFN layer for
 * MI355X (gfx950).
 *
 * The layer is the routed MoE FFN of a Hunyuan-Image-3.0-style transformer as
 * described in "Hunyuan Image 3.0 hybrid parallelism" (LightX2V blog), section
 * 6 (multi-micro-shard fused MoE): a router yields expert ids and routing
 * scores per token; the flattened ids are sorted by expert into a route
 * permutation with per-expert offsets; the input is indexed once by that
 * permutation; every micro-shard runs a grouped gate|up GEMM, SwiGLU and a
 * grouped down GEMM; one finalize applies the routing scale and reduces the
 * top-k routes once.  Expert semantics down(SiLU(gate(x)) * up(x)) with gate
 * and up fused as one w13 weight follow "HunyuanImage-3.0 on CANN NPU",
 * section 2.2.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers to caller-owned memory, 16-byte
 *    aligned, row-major and contiguous.  The library never allocates or frees
 *    device memory and keeps no state between calls; calls on distinct
 *    buffers are independent.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on it and returns; nothing is read back to the
 *    host and nothing synchronises.
 *  - Arguments are validated on the host first.  On any error nothing is
 *    enqueued and no output is touched.  Device data (finite logits and
 *    weights) is a documented precondition, not checked.
 *  - A shape with T == 0 is valid: the call validates and enqueues nothing,
 *    except moe_permute, which writes zero counts and offsets.
 *
 * Notation: T tokens, H hidden size, E experts, k routes per token,
 * Im intermediate columns per micro-shard, mu = micro_count, R = T*k routes.
 * dtype is the element type of x, w1, w2, h and out (MOE_BF16 or MOE_F32);
 * router weights, bias, logits and routing weights are always fp32.
 *
 * y, the down projection's output [rows, H] that the finalize consumes, is
 * fp32 in an MOE_F32 layer.  In an MOE_BF16 layer it is "block-scaled half":
 * each row is cut into blocks of MOE_Y_BLOCK columns; the buffer holds the
 * values as fp16 [rows, H] followed by one int8 exponent per block
 * [rows, ceil(H / MOE_Y_BLOCK)] (the last block of a row is partial when
 * H % MOE_Y_BLOCK != 0), and y[p, n] = value[p, n] * 2^exponent[p, n / MOE_Y_BLOCK].
 * A block's exponent is floor(log2 M) - 14 for its largest magnitude M (0 for
 * an all-zero block), so every value keeps 11 significant bits in the bytes of
 * bf16 plus one per block.  (A bf16 y would be a third rounding between the
 * fp32 accumulator and the output; at outputs of magnitude 4 and more that
 * takes the error past the bf16 bar of 2e-2.)  Size: MOE_Y_BYTES(dtype, rows, H).
 *
 * Envelope (MOE_ERR_UNSUPPORTED outside it): 1 <= E <= 64, H % 64 == 0,
 * Im % 32 == 0, R < 2^31, every size in elements < 2^31, one expert's w1
 * block (2*Im*H elements of 2 bytes) < 4 GiB.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* negative or inconsistent sizes, null pointer, bad dtype */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but outside the envelope above, or misaligned */
  MOE_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than moe_workspace_size */
  MOE_ERR_HIP = 4           /* a HIP launch reported an error */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Columns per exponent of a block-scaled half y, and the bytes of a y buffer. */
#define MOE_Y_BLOCK 256
#define MOE_Y_BYTES(dtype, rows, H)                                                        \
  ((dtype) == MOE_BF16 ? (size_t)(rows) * (size_t)(H) * 2 + (size_t)(rows) * (((H) + MOE_Y_BLOCK - 1) / MOE_Y_BLOCK) \
                       : (size_t)(rows) * (size_t)(H) * 4)

typedef struct {
  int32_t T;            /* tokens, >= 0 */
  int32_t H;            /* hidden size */
  int32_t E;            /* experts, 1..64 */
  int32_t k;            /* routes per token, 1..E */
  int32_t Im;           /* intermediate columns per micro-shard */
  int32_t micro_count;  /* micro-shards stored micro-major, >= 1 */
  int32_t dtype;        /* moe_dtype */
  int32_t renormalize;  /* 1: routing weights renormalised to sum 1 over the k selected
                           experts; 0: the softmax over all E experts at the selected ones */
} moe_shape;

/* Byte offsets of the intermediates inside a moe_forward workspace (each
 * 256-byte aligned), so a caller can inspect them after the call. */
typedef struct {
  size_t logits;   /* float   [T, E]         */
  size_t topk_ids; /* int32   [T, k]         */
  size_t topk_w;   /* float   [T, k]         */
  size_t counts;   /* int32   [E]            */
  size_t offsets;  /* int32   [E + 1]        */
  size_t perm;     /* int32   [R]            */
  size_t inv;      /* int32   [R]            */
  size_t h;        /* dtype   [R, mu*Im]     */
  size_t y;        /* y       [R, H] (fp32, or block-scaled half for bf16) */
  size_t scratch;  /* token path: int32 [ceil(T/16), 64] expert counts per 16-token router
                      block; small-token path: fp64 router partials, active-expert list */
  size_t total;    /* bytes needed            */
} moe_workspace_layout;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status s);

/* Workspace bytes that moe_forward needs for `shape`, or 0 if the shape is
 * invalid or unsupported.  Pure host function. */
size_t moe_workspace_size(const moe_shape* shape);

/* Fills `layout` for `shape`.  Pure host function. */
moe_status moe_get_workspace_layout(const moe_shape* shape, moe_workspace_layout* layout);

/* Router and gating (hybrid parallelism, section 6.1: ids and routing scores
 * of shape [num_tokens, top_k]; CANN NPU, section 5.2: the gate in fp32).
 *   x [T, H] dtype; wg [E, H] fp32; bias [E] fp32 or NULL.
 *   logits[t, e] = fp32(sum_h double(x[t,h]) * double(wg[e,h]) + double(bias[e])):
 *     products and sum in fp64, one rounding to fp32.
 *   topk_ids[t, j]: the j-th expert in (logit descending, expert ascending)
 *     order, -0.0 equal to +0.0; topk_w[t, j] = softmax over all experts at
 *     the selected ones (computed in fp64, rounded once), renormalised to sum
 *     1 over the k selected when shape->renormalize is 1.
 * Outputs: logits [T, E] fp32, topk_ids [T, k] int32, topk_w [T, k] fp32. */
moe_status moe_route(const moe_shape* shape, const void* x, const float* wg, const float* bias,
                     float* logits, int32_t* topk_ids, float* topk_w, void* stream);

/* Route permutation and expert offsets (hybrid parallelism, section 6.1:
 * sort the flattened ids by expert into permuted_to_expanded, bincount then
 * cumsum for the offsets; the inverse permutation for finalize).
 *   counts[e] = number of routes to expert e; offsets [E + 1] exclusive
 *   (offsets[0] = 0, offsets[E] = R); perm[p] = route r = t*k + j of permuted
 *   row p, stable (rows of one expert in increasing r); inv[perm[p]] = p.
 *   If both x and permuted_x are non-NULL, also writes the gathered input
 *   permuted_x[p, :] = x[perm[p] / k, :] (dtype, [R, H]); the one-call path
 *   never materialises it (the w13 GEMM gathers rows itself).
 * With T == 0 only counts and offsets are written (all zero); the other
 * pointers may then be NULL.
 * topk_ids must hold experts in [0, E) (as moe_route writes them); an id
 * outside that range is clamped into it, so every write stays in bounds and
 * perm is still a permutation, but the result is then unspecified.
 * Deterministic and atomic-free in its outputs. */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv,
                       const void* x, void* permuted_x, void* stream);

/* Grouped gate|up GEMM with the SwiGLU epilogue, all micro-shards in one
 * launch (hybrid parallelism, section 6.1: grouped GEMM1, split gate/up,
 * SiLU * mul; CANN NPU, section 2.2: SiLU on the gate half times the up half).
 *   w1 [mu, E, 2*Im, H] dtype, micro-major; in w1[m][e] rows [0, Im) are gate
 *   and rows [Im, 2*Im) the matching up rows.
 *   h[p, m*Im + i] = SiLU(g) * u with g = x[perm[p]/k] . w1[m][e][i],
 *   u = x[perm[p]/k] . w1[m][e][Im + i], e the expert whose offsets segment
 *   holds p; fp32 accumulation, SiLU(z) = z / (1 + e^-z), one rounding to
 *   dtype.  Output h [R, mu*Im] dtype.
 *   perm and offsets must be moe_permute's outputs for this shape (offsets
 *   non-decreasing from 0 to R, perm a permutation of [0, R)): the kernels
 *   index with them unchecked. */
moe_status moe_grouped_gemm_w13_swiglu(const moe_shape* shape, const void* x, const int32_t* perm,
                                       const int32_t* offsets, const void* w1, void* h,
                                       void* stream);

/* Grouped down GEMM with micro-shards summed in the accumulator (hybrid
 * parallelism, section 6.1: grouped GEMM2 per micro, partials added in fp32).
 *   w2 [mu, E, H, Im] dtype, micro-major.
 *   y[p, n] = sum_m sum_i h[p, m*Im + i] * w2[m][e][n][i], fp32 accumulation.
 *   Output y [R, H]: fp32 (MOE_F32), block-scaled half (MOE_BF16; see above),
 *   MOE_Y_BYTES(dtype, R, H) bytes.  offsets as for the w13 GEMM
 *   (moe_permute's, used unchecked). */
moe_status moe_grouped_gemm_down(const moe_shape* shape, const void* h, const int32_t* offsets,
                                 const void* w2, void* y, void* stream);

/* Finalize: routing scale and top-k reduction once (hybrid parallelism,
 * section 6.1, the finalize formula).
 *   out[t, :] = sum_{j = 0..k-1} topk_w[t, j] * y[inv[t*k + j], :], fp32,
 *   j ascending, one rounding to dtype.  y [R, H] as moe_grouped_gemm_down
 *   writes it.  Output out [T, H] dtype.  inv must be moe_permute's (values in
 *   [0, R), used unchecked). */
moe_status moe_finalize(const moe_shape* shape, const void* y, const int32_t* inv,
                        const float* topk_w, void* out, void* stream);

/* The whole layer in one call: route, permute, grouped w13+SwiGLU, grouped
 * down, finalize, sharing one permutation and one set of offsets across all
 * micro-shards and finalizing once (hybrid parallelism, section 6: the
 * multi-micro-shard fused MoE).  micro_count = 1 covers an expert-major
 * shard and a single micro view (pass w1/w2 offset to that micro).
 *   workspace: device buffer of at least moe_workspace_size(shape) bytes,
 *   256-byte aligned; its intermediates sit at moe_get_workspace_layout's
 *   offsets.
 *   Small token counts (T <= 16, bf16, H % 2048 == 0, Im % 256 == 0) take a
 *   weight-streaming path (the AR-decode regime: hybrid parallelism,
 *   sections 4.3 and 6.2): routing, counts, offsets, perm and inv are the
 *   same bits as the step-wise path, h is computed the same way, and the down
 *   projection is fused with the finalize (y is never written; its fp32 values
 *   are summed unrounded and in another order), so the output matches the
 *   step-wise path within rounding, not bit for bit; the y region is then
 *   left untouched.
 *   Output out [T, H] dtype. */
moe_status moe_forward(const moe_shape* shape, const void* x, const float* wg, const float* bias,
                       const void* w1, const void* w2, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same layer and launch sequence as moe_forward, with the workspace
 * taken from a static device array of MOE_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds on each GPU it runs on until the process ends (set up on
 * the first call on a device, which must be the current device; no
 * hipMalloc, hipFree or other allocation, ever).  Inputs and output are the
 * caller's, as for moe_forward.
 *   Shapes whose moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES (the
 *   small-token regime fits: the decode layer T=8, H=4096, E=64, k=8, Im=768
 *   needs under 1 MiB) are rejected with MOE_ERR_WORKSPACE before anything is
 *   enqueued.
 *   Every call on one GPU uses that GPU's one array and leaves the call's
 *   intermediates in it: calls that may overlap on one GPU (other streams,
 *   other threads) race and must be serialised by the caller.  No kernel of
 *   the call needs the array cleared beforehand. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* wg,
                               const float* bias, const void* w1, const void* w2, void* out,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
