// C ABI of the MoE library: host-side validation, workspace layout and the
// launch sequence.  Declarations and argument semantics: moe_mi355x.h and,
// for the shared expert, moe_shared.h.
//
// Every entry point validates everything it can on the host before any HIP
// call, so a rejected call enqueues nothing and touches no output.
#include "../../include/moe_mi355x.h"
#include "../../include/moe_shared.h"
#include "moe_common.h"

#include <algorithm>
#include <mutex>

using moe::Shape;

// Scratch of moe_forward_noalloc: one copy per GPU, held until the process
// ends.  In host code this name is only a stand-in for the symbol; the device
// address of each GPU's copy comes from hipGetSymbolAddress (noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by every entry point.
moe_status check_shape(const moe_shape* sh, Shape* out) {
  if (sh == nullptr) return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *sh;
  if (s.T < 0 || s.H <= 0 || s.E <= 0 || s.k <= 0 || s.Im <= 0 || s.micro_count <= 0)
    return MOE_ERR_INVALID_ARG;
  if (s.k > s.E) return MOE_ERR_INVALID_ARG;
  if (s.dtype != MOE_F32 && s.dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.renormalize != 0 && s.renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (s.E > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  // k-steps of 64 over H (w13) and of 32 over Im (down); w13 output tiles of
  // 32 columns; down output tiles of 64 columns (the fp32 path)
  if (s.H % 64 != 0 || s.Im % 32 != 0) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)s.T * s.k;
  const long long I = (long long)s.micro_count * s.Im;
  const long long lim = (1ll << 31) - 1;
  // the GEMMs address one expert's weight block (w1: 2*Im x H, w2: H x Im)
  // with 32-bit byte offsets
  const long long expert_w1_bytes = 4ll * s.Im * s.H;
  if (R > lim || I > lim || R * s.H > lim || R * I > lim || (long long)s.T * s.H > lim ||
      (long long)s.micro_count * s.E * 2 * s.Im * s.H > lim * 8 || expert_w1_bytes > 0xffffffffll)
    return MOE_ERR_UNSUPPORTED;
  if (out) {
    out->T = s.T; out->H = s.H; out->E = s.E; out->k = s.k; out->Im = s.Im;
    out->mu = s.micro_count; out->bf16 = (s.dtype == MOE_BF16);
    out->renorm = (s.renormalize != 0);
  }
  return MOE_OK;
}

// Non-null and 16-byte aligned (the kernels move 16-byte vectors).
moe_status check_ptr(const void* p) {
  if (p == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

#define MOE_CHECK(expr)                 \
  do {                                  \
    const moe_status st_ = (expr);      \
    if (st_ != MOE_OK) return st_;      \
  } while (0)

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

inline size_t elem_bytes(const Shape& s) { return s.bf16 ? 2 : 4; }

static_assert(moe::kYBlock == MOE_Y_BLOCK, "y block of the header and the kernels");

// A y buffer of `rows` rows: fp32 in the fp32 layer, block-scaled half in the
// bf16 layers (moe_common.h).
inline size_t y_bytes(const Shape& s, long long rows) {
  return s.bf16 ? moe::y_half_bytes(rows, s.H) : (size_t)rows * s.H * 4;
}

void layout_of(const Shape& s, moe_workspace_layout* L) {
  const size_t R = (size_t)s.R();
  size_t o = 0;
  L->logits = o;   o = align_up(o + (size_t)s.T * s.E * 4);
  L->topk_ids = o; o = align_up(o + R * 4);
  L->topk_w = o;   o = align_up(o + R * 4);
  L->counts = o;   o = align_up(o + (size_t)s.E * 4);
  L->offsets = o;  o = align_up(o + (size_t)(s.E + 1) * 4);
  L->perm = o;     o = align_up(o + R * 4);
  L->inv = o;      o = align_up(o + R * 4);
  L->h = o;        o = align_up(o + R * (size_t)s.mu * s.Im * elem_bytes(s));
  L->y = o;        o = align_up(o + y_bytes(s, s.R()));
  L->scratch = o;
  o = align_up(o + std::max(moe::decode_scratch_bytes(), moe::route_hist_bytes(s)));
  L->total = o;
}

// The shared expert's width against the envelope (moe_shared.h).
moe_status check_shared(const Shape& s, int32_t Is) {
  if (Is <= 0) return MOE_ERR_INVALID_ARG;
  if (Is % 32 != 0) return MOE_ERR_UNSUPPORTED;
  const long long lim = (1ll << 31) - 1;
  if ((long long)s.T * Is > lim || 2ll * Is * s.H > lim || 4ll * Is * s.H > 0xffffffffll)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// moe_forward's workspace, then hs [T, Is] and ys [T, H].
void shared_layout_of(const Shape& s, int Is, moe_shared_layout* L) {
  moe_workspace_layout base;
  layout_of(s, &base);
  size_t o = base.total;
  L->hs = o; o = align_up(o + (size_t)s.T * Is * elem_bytes(s));
  L->ys = o; o = align_up(o + y_bytes(s, s.T));
  L->total = o;
}

// The shared expert as the grouped GEMMs see it: one expert, one route per
// token, one micro of width Is; its launches pass no offsets (one dense
// segment of the T tokens in order).
Shape dense_shape(const Shape& s, int Is) {
  Shape d = s;
  d.E = 1;
  d.k = 1;
  d.Im = Is;
  d.mu = 1;
  return d;
}

struct SharedArgs {
  int Is;
  const void* w1s;
  const void* w2s;
  moe_shared_layout L;
};

// moe_forward and moe_forward_shared (sh == nullptr: no shared expert).
moe_status forward_impl(const Shape& s, const void* x, const float* wg, const float* bias,
                        const void* w1, const void* w2, void* out, void* workspace,
                        size_t workspace_bytes, hipStream_t st, const SharedArgs* sh) {
  moe_workspace_layout L;
  layout_of(s, &L);
  const size_t need = sh ? sh->L.total : L.total;
  if (workspace == nullptr || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MOE_ERR_UNSUPPORTED;

  char* ws = (char*)workspace;
  float* logits = (float*)(ws + L.logits);
  int32_t* ids = (int32_t*)(ws + L.topk_ids);
  float* w = (float*)(ws + L.topk_w);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* perm = (int32_t*)(ws + L.perm);
  int32_t* inv = (int32_t*)(ws + L.inv);
  void* h = ws + L.h;
  void* y = ws + L.y;

  if (moe::decode_supported(s) && (sh == nullptr || moe::decode_shared_supported(sh->Is))) {
    moe::SharedExpert se;
    if (sh) se = moe::SharedExpert{sh->w1s, sh->w2s, sh->Is, ws + sh->L.hs};
    return hip_status(moe::launch_decode(s, x, wg, bias, w1, w2, out, logits, ids, w, counts,
                                         offsets, perm, inv, h, ws + L.scratch, st,
                                         sh ? &se : nullptr));
  }
  int32_t* hist = (int32_t*)(ws + L.scratch);
  MOE_CHECK(hip_status(moe::launch_route(s, x, wg, bias, logits, ids, w, st, hist)));
  MOE_CHECK(hip_status(moe::launch_permute_hist(s, ids, hist, counts, offsets, perm, inv, st)));
  void* ys = nullptr;
  if (sh && s.bf16) {
    // the shared expert's tiles ride in the routed GEMMs' launches (its w13
    // alone would leave part of the device idle)
    void* hs = ws + sh->L.hs;
    ys = ws + sh->L.ys;
    MOE_CHECK(hip_status(
        moe::launch_w13_swiglu_with_dense(s, x, perm, offsets, w1, h, sh->w1s, hs, sh->Is, st)));
    MOE_CHECK(hip_status(
        moe::launch_down_with_dense(s, h, offsets, w2, y, hs, sh->w2s, ys, sh->Is, st)));
  } else {
    MOE_CHECK(hip_status(moe::launch_w13_swiglu(s, x, perm, offsets, w1, h, st)));
    MOE_CHECK(hip_status(moe::launch_down(s, h, offsets, w2, y, st)));
    if (sh) {
      const Shape d = dense_shape(s, sh->Is);
      void* hs = ws + sh->L.hs;
      ys = ws + sh->L.ys;
      MOE_CHECK(hip_status(moe::launch_w13_swiglu(d, x, nullptr, nullptr, sh->w1s, hs, st)));
      MOE_CHECK(hip_status(moe::launch_down(d, hs, nullptr, sh->w2s, ys, st)));
    }
  }
  MOE_CHECK(hip_status(moe::launch_finalize(s, y, inv, w, out, st, ys)));
  return MOE_OK;
}

// Device address of the current GPU's copy of `scratch`, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the supported envelope or misaligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
  }
  return "unknown moe_status";
}

size_t moe_workspace_size(const moe_shape* shape) {
  Shape s;
  if (check_shape(shape, &s) != MOE_OK) return 0;
  moe_workspace_layout L;
  layout_of(s, &L);
  return L.total;
}

moe_status moe_get_workspace_layout(const moe_shape* shape, moe_workspace_layout* layout) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (layout == nullptr) return MOE_ERR_INVALID_ARG;
  layout_of(s, layout);
  return MOE_OK;
}

moe_status moe_route(const moe_shape* shape, const void* x, const float* wg, const float* bias,
                     float* logits, int32_t* topk_ids, float* topk_w, void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x)); MOE_CHECK(check_ptr(wg)); MOE_CHECK(check_ptr(logits));
  MOE_CHECK(check_ptr(topk_ids)); MOE_CHECK(check_ptr(topk_w));
  if (bias != nullptr) MOE_CHECK(check_ptr(bias));
  return hip_status(moe::launch_route(s, x, wg, bias, logits, topk_ids, topk_w, (hipStream_t)stream));
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, const void* x,
                       void* permuted_x, void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  MOE_CHECK(check_ptr(counts)); MOE_CHECK(check_ptr(offsets));
  if ((x == nullptr) != (permuted_x == nullptr)) return MOE_ERR_INVALID_ARG;
  if (s.T == 0)  // no routes: zero counts and offsets, nothing else
    return hip_status(moe::launch_permute(s, topk_ids, counts, offsets, perm, inv, (hipStream_t)stream));
  MOE_CHECK(check_ptr(topk_ids)); MOE_CHECK(check_ptr(perm)); MOE_CHECK(check_ptr(inv));
  if (x != nullptr) { MOE_CHECK(check_ptr(x)); MOE_CHECK(check_ptr(permuted_x)); }
  hipStream_t st = (hipStream_t)stream;
  MOE_CHECK(hip_status(moe::launch_permute(s, topk_ids, counts, offsets, perm, inv, st)));
  if (x != nullptr) MOE_CHECK(hip_status(moe::launch_gather(s, x, perm, permuted_x, st)));
  return MOE_OK;
}

moe_status moe_grouped_gemm_w13_swiglu(const moe_shape* shape, const void* x, const int32_t* perm,
                                       const int32_t* offsets, const void* w1, void* h,
                                       void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x)); MOE_CHECK(check_ptr(perm)); MOE_CHECK(check_ptr(offsets));
  MOE_CHECK(check_ptr(w1)); MOE_CHECK(check_ptr(h));
  return hip_status(moe::launch_w13_swiglu(s, x, perm, offsets, w1, h, (hipStream_t)stream));
}

moe_status moe_grouped_gemm_down(const moe_shape* shape, const void* h, const int32_t* offsets,
                                 const void* w2, void* y, void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(h)); MOE_CHECK(check_ptr(offsets)); MOE_CHECK(check_ptr(w2));
  MOE_CHECK(check_ptr(y));
  return hip_status(moe::launch_down(s, h, offsets, w2, y, (hipStream_t)stream));
}

moe_status moe_finalize(const moe_shape* shape, const void* y, const int32_t* inv,
                        const float* topk_w, void* out, void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(y)); MOE_CHECK(check_ptr(inv)); MOE_CHECK(check_ptr(topk_w));
  MOE_CHECK(check_ptr(out));
  return hip_status(moe::launch_finalize(s, y, inv, topk_w, out, (hipStream_t)stream));
}

moe_status moe_forward(const moe_shape* shape, const void* x, const float* wg, const float* bias,
                       const void* w1, const void* w2, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x)); MOE_CHECK(check_ptr(wg)); MOE_CHECK(check_ptr(w1));
  MOE_CHECK(check_ptr(w2)); MOE_CHECK(check_ptr(out));
  if (bias != nullptr) MOE_CHECK(check_ptr(bias));
  return forward_impl(s, x, wg, bias, w1, w2, out, workspace, workspace_bytes, (hipStream_t)stream,
                      nullptr);
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* wg,
                               const float* bias, const void* w1, const void* w2, void* out,
                               void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x)); MOE_CHECK(check_ptr(wg)); MOE_CHECK(check_ptr(w1));
  MOE_CHECK(check_ptr(w2)); MOE_CHECK(check_ptr(out));
  if (bias != nullptr) MOE_CHECK(check_ptr(bias));
  moe_workspace_layout L;
  layout_of(s, &L);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  MOE_CHECK(noalloc_scratch(&ws));
  // the same launch sequence as moe_forward, on the device's static scratch
  // (no kernel of it needs the workspace cleared first)
  return forward_impl(s, x, wg, bias, w1, w2, out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                      (hipStream_t)stream, nullptr);
}

// ---- shared expert (moe_shared.h)

size_t moe_shared_workspace_size(const moe_shape* shape, int32_t Is) {
  Shape s;
  if (check_shape(shape, &s) != MOE_OK || check_shared(s, Is) != MOE_OK) return 0;
  moe_shared_layout L;
  shared_layout_of(s, Is, &L);
  return L.total;
}

moe_status moe_get_shared_workspace_layout(const moe_shape* shape, int32_t Is,
                                           moe_shared_layout* layout) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  MOE_CHECK(check_shared(s, Is));
  if (layout == nullptr) return MOE_ERR_INVALID_ARG;
  shared_layout_of(s, Is, layout);
  return MOE_OK;
}

moe_status moe_shared_ffn(const moe_shape* shape, int32_t Is, const void* x, const void* w1s,
                          const void* w2s, void* hs, void* ys, void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  MOE_CHECK(check_shared(s, Is));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x)); MOE_CHECK(check_ptr(w1s)); MOE_CHECK(check_ptr(w2s));
  MOE_CHECK(check_ptr(hs)); MOE_CHECK(check_ptr(ys));
  hipStream_t st = (hipStream_t)stream;
  const Shape d = dense_shape(s, Is);
  MOE_CHECK(hip_status(moe::launch_w13_swiglu(d, x, nullptr, nullptr, w1s, hs, st)));
  return hip_status(moe::launch_down(d, hs, nullptr, w2s, ys, st));
}

moe_status moe_finalize_shared(const moe_shape* shape, const void* y, const int32_t* inv,
                               const float* topk_w, const void* ys, void* out, void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(y)); MOE_CHECK(check_ptr(inv)); MOE_CHECK(check_ptr(topk_w));
  MOE_CHECK(check_ptr(ys)); MOE_CHECK(check_ptr(out));
  return hip_status(moe::launch_finalize(s, y, inv, topk_w, out, (hipStream_t)stream, ys));
}

moe_status moe_forward_shared(const moe_shape* shape, int32_t Is, const void* x, const float* wg,
                              const float* bias, const void* w1, const void* w2, const void* w1s,
                              const void* w2s, void* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Shape s;
  MOE_CHECK(check_shape(shape, &s));
  MOE_CHECK(check_shared(s, Is));
  if (s.T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x)); MOE_CHECK(check_ptr(wg)); MOE_CHECK(check_ptr(w1));
  MOE_CHECK(check_ptr(w2)); MOE_CHECK(check_ptr(w1s)); MOE_CHECK(check_ptr(w2s));
  MOE_CHECK(check_ptr(out));
  if (bias != nullptr) MOE_CHECK(check_ptr(bias));
  SharedArgs sh;
  sh.Is = Is;
  sh.w1s = w1s;
  sh.w2s = w2s;
  shared_layout_of(s, Is, &sh.L);
  return forward_impl(s, x, wg, bias, w1, w2, out, workspace, workspace_bytes, (hipStream_t)stream,
                      &sh);
}

}  // extern "C"
