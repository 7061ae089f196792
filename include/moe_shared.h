/*
 * moe_shared.h -- the shared expert beside the routed experts, C ABI.
 *
 * "HunyuanImage-3.0 on CANN NPU", section 3.1: besides the routed experts
 * (deployed tensor-parallel) every token also passes through a shared expert,
 * whose computation that page overlaps with the communication that follows
 * the routed experts (on a second stream).  The pages give no shape for the
 * shared expert and no gate on its output.  This library takes the plainest
 * reading: a SwiGLU expert of the same form as the routed ones (CANN NPU,
 * section 2.2: down(SiLU(gate(x)) * up(x)), gate and up fused as one w13
 * weight), applied to every token, its output added to the routed output
 * with weight 1:
 *
 *   out[t, :] = sum_{j ascending} topk_w[t, j] * y[inv[t*k + j], :] + ys[t, :]
 *   ys[t, n]  = sum_i hs[t, i] * w2s[n, i]
 *   hs[t, i]  = SiLU(x[t] . w1s[i]) * (x[t] . w1s[Is + i])
 *
 * Is is the shared expert's intermediate width on this rank (a tensor-
 * parallel shard of it, like the routed experts' Im).
 *
 * Conventions are those of moe_mi355x.h: device pointers to caller-owned,
 * 16-byte aligned, contiguous row-major memory; `stream` is a hipStream_t
 * passed as void*; host-side validation first, and on any error nothing is
 * enqueued and no output is touched; T == 0 is valid and enqueues nothing.
 *
 * Layouts: w1s [2*Is, H] dtype, rows [0, Is) gate and [Is, 2*Is) the
 * matching up rows; w2s [H, Is] dtype; hs [T, Is] dtype; ys [T, H] in the
 * format of the routed y (moe_mi355x.h: fp32, or block-scaled half in a bf16
 * layer; MOE_Y_BYTES(dtype, T, H) bytes).  Sums are in fp32 and every dtype
 * result is rounded once.
 *
 * Envelope, beside moe_mi355x.h's: Is % 32 == 0, T*Is < 2^31, the w1s block
 * (2*Is*H elements of 2 bytes) < 4 GiB; otherwise MOE_ERR_UNSUPPORTED.
 * Is <= 0 is MOE_ERR_INVALID_ARG.
 */
#ifndef MOE_SHARED_H
#define MOE_SHARED_H

#include "moe_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Byte offsets of the shared expert's regions in a moe_forward_shared
 * workspace.  The workspace starts with exactly the moe_forward workspace
 * of the same shape (moe_get_workspace_layout's offsets hold unchanged);
 * the shared regions follow it, each 256-byte aligned. */
typedef struct {
  size_t hs;     /* dtype [T, Is]: the shared expert's SwiGLU activations */
  size_t ys;     /* y format [T, H]: its output (token path only; the small-token
                    path fuses it into the output and leaves this region alone) */
  size_t total;  /* bytes needed */
} moe_shared_layout;

/* Workspace bytes moe_forward_shared needs, or 0 if shape or Is is invalid
 * or unsupported.  Pure host function. */
size_t moe_shared_workspace_size(const moe_shape* shape, int32_t Is);

/* Fills `layout` for (shape, Is).  Pure host function. */
moe_status moe_get_shared_workspace_layout(const moe_shape* shape, int32_t Is,
                                           moe_shared_layout* layout);

/* The shared expert over all T tokens, step-wise: the grouped w13+SwiGLU and
 * down GEMMs of moe_mi355x.h run on one dense segment of the T tokens in
 * order.
 *   x [T, H], w1s [2*Is, H], w2s [H, Is] (dtype).
 * Outputs: hs [T, Is] (dtype) and ys [T, H] (y format). */
moe_status moe_shared_ffn(const moe_shape* shape, int32_t Is, const void* x, const void* w1s,
                          const void* w2s, void* hs, void* ys, void* stream);

/* moe_finalize plus the shared expert's output: the routed sum over j
 * ascending in fp32, then + ys[t, :], one rounding.
 *   y [R, H] and ys [T, H] (y format), inv [R] int32, topk_w [T, k] fp32.
 * Output: out [T, H] dtype. */
moe_status moe_finalize_shared(const moe_shape* shape, const void* y, const int32_t* inv,
                               const float* topk_w, const void* ys, void* out, void* stream);

/* The whole layer with its shared expert in one call: moe_forward's routed
 * path, the shared expert's two GEMMs, and one finalize that adds it.
 *   workspace: at least moe_shared_workspace_size(shape, Is) bytes, 256-byte
 *   aligned.
 *   Small token counts on moe_forward's weight-streaming path (and
 *   Is % 256 == 0) stream the shared expert's weights in the same two
 *   launches as the routed experts' and add its output inside the fused
 *   down+finalize (hs is written, ys is not).  Output out [T, H] dtype. */
moe_status moe_forward_shared(const moe_shape* shape, int32_t Is, const void* x, const float* wg,
                              const float* bias, const void* w1, const void* w2, const void* w1s,
                              const void* w2s, void* out, void* workspace, size_t workspace_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SHARED_H */
