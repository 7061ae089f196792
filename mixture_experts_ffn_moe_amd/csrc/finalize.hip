// Finalize: routing scale and top-k reduction, once per token.
//
// "Hunyuan Image 3.0 hybrid parallelism", section 6.1: finalize reads the
// expert outputs by original token and top-k slot through the inverse
// permutation, applies the routing score once and reduces the top-k routes
// once.  The micro-shard partials were already summed in the down GEMM's fp32
// accumulator, so each route contributes one row of y: fp32 in the fp32 layer,
// block-scaled half (11 significant bits, moe_common.h) in the bf16 layers.
//
// out[t, :] = sum_{j ascending} w[t, j] * y[inv[t*k + j], :] in fp32, one
// rounding.  With a shared expert ("HunyuanImage-3.0 on CANN NPU", section
// 3.1: every token also passes through a shared expert whose output joins the
// routed experts' sum) its output row ys[t, :] is added after the routed sum,
// before the rounding.  No atomics: every output element is owned by one thread, so the
// result is bitwise reproducible.  One workgroup per token; each thread moves
// 16-byte vectors, so every row read is fully coalesced.
#include "moe_common.h"

namespace moe {
namespace {

// One route row's 8 columns [c, c + 8) as fp32: fp32 y (the fp32 layer) or
// block-scaled half y (the bf16 layers; values plane `y`, exponents `ye`).
struct YRow {
  __device__ __forceinline__ static void load(const float* y, const int8_t*, size_t row, int H, int c,
                                              float (&v)[8]) {
    const float4* src = reinterpret_cast<const float4*>(y + row * H + c);
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void load(const _Float16* y, const int8_t* ye, size_t row, int H, int c,
                                              float (&v)[8]) {
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    const f16x8 h = *reinterpret_cast<const f16x8*>(y + row * H + c);
    const int e = ye[row * ((H + kYBlock - 1) / kYBlock) + c / kYBlock];  // a partial last block when H % kYBlock != 0
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = ldexpf((float)h[q], e);
  }
};

// out has the layer's element type T; y and ys are fp32 for the fp32 layer
// and block-scaled half (values YT = _Float16 plus int8 exponents) for the
// bf16 layers.  A thread owns 8 consecutive columns (within one y block).
template <typename T, typename YT>
__global__ __launch_bounds__(256) void finalize_kernel(const YT* __restrict__ y,
                                                       const int8_t* __restrict__ ye,
                                                       const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w,
                                                       const YT* __restrict__ ys,
                                                       const int8_t* __restrict__ yse, int H, int k,
                                                       T* __restrict__ out) {
  constexpr int V = 8;  // columns per thread
  const int t = blockIdx.x;
  const int32_t* rows = inv + (size_t)t * k;
  const float* wt = w + (size_t)t * k;
  for (int c = threadIdx.x * V; c < H; c += blockDim.x * V) {
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.0f;
    // routes in groups of 4: a group's row loads are all in flight before the
    // first is used; the sum still runs over j ascending
    int j = 0;
    for (; j + 4 <= k; j += 4) {
      float v[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u) YRow::load(y, ye, (size_t)rows[j + u], H, c, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float s = wt[j + u];
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] = fmaf(s, v[u][q], acc[q]);
      }
    }
    for (; j < k; ++j) {
      float v[V];
      YRow::load(y, ye, (size_t)rows[j], H, c, v);
      const float s = wt[j];
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = fmaf(s, v[q], acc[q]);
    }
    if (ys != nullptr) {
      float v[V];
      YRow::load(ys, yse, (size_t)t, H, c, v);
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] += v[q];
    }
    alignas(16) T res[V];
#pragma unroll
    for (int q = 0; q < V; ++q) res[q] = Elem<T>::from_f(acc[q]);
    uint4* dst = reinterpret_cast<uint4*>(out + (size_t)t * H + c);
#pragma unroll
    for (int q = 0; q < V * (int)sizeof(T) / 16; ++q) dst[q] = reinterpret_cast<const uint4*>(res)[q];
  }
}

}  // namespace

hipError_t launch_finalize(const Shape& s, const void* y, const int32_t* inv, const float* w,
                           void* out, hipStream_t st, const void* ys) {
  if (s.bf16) {
    // block-scaled half: the exponent plane follows the values plane
    const int8_t* ye = (const int8_t*)y + (size_t)s.R() * s.H * 2;
    const int8_t* yse = ys ? (const int8_t*)ys + (size_t)s.T * s.H * 2 : nullptr;
    hipLaunchKernelGGL((finalize_kernel<uint16_t, _Float16>), dim3(s.T), dim3(256), 0, st,
                       (const _Float16*)y, ye, inv, w, (const _Float16*)ys, yse, s.H, s.k,
                       (uint16_t*)out);
  } else {
    hipLaunchKernelGGL((finalize_kernel<float, float>), dim3(s.T), dim3(256), 0, st, (const float*)y,
                       (const int8_t*)nullptr, inv, w, (const float*)ys, (const int8_t*)nullptr, s.H,
                       s.k, (float*)out);
  }
  return hipGetLastError();
}

}  // namespace moe
