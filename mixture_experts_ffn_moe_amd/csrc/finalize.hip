// Finalize: routing scale and top-k reduction, once per token.
//
// "Hunyuan Image 3.0 hybrid parallelism", section 6.1: finalize reads the
// expert outputs by original token and top-k slot through the inverse
// permutation, applies the routing score once and reduces the top-k routes
// once.  The micro-shard partials were already summed in the down GEMM's fp32
// accumulator, so each route contributes one row of y.
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

template <typename T>
__global__ __launch_bounds__(256) void finalize_kernel(const T* __restrict__ y,
                                                       const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w,
                                                       const T* __restrict__ ys, int H, int k,
                                                       T* __restrict__ out) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector
  const int t = blockIdx.x;
  const int32_t* rows = inv + (size_t)t * k;
  const float* wt = w + (size_t)t * k;
  for (int c = threadIdx.x * V; c < H; c += blockDim.x * V) {
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.0f;
    // routes in groups of 8: a group's row loads are all in flight before the
    // first is used (7% faster than one at a time); the sum still runs over j
    // ascending
    int j = 0;
    for (; j + 8 <= k; j += 8) {
      uint4 raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = *reinterpret_cast<const uint4*>(y + (size_t)rows[j + u] * H + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float s = wt[j + u];
        const T* v = reinterpret_cast<const T*>(&raw[u]);
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] = fmaf(s, Elem<T>::to_f(v[q]), acc[q]);
      }
    }
    for (; j < k; ++j) {
      const float s = wt[j];
      const uint4 raw = *reinterpret_cast<const uint4*>(y + (size_t)rows[j] * H + c);
      const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = fmaf(s, Elem<T>::to_f(v[q]), acc[q]);
    }
    if (ys != nullptr) {
      const uint4 raw = *reinterpret_cast<const uint4*>(ys + (size_t)t * H + c);
      const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] += Elem<T>::to_f(v[q]);
    }
    uint4 res;
    T* o = reinterpret_cast<T*>(&res);
#pragma unroll
    for (int q = 0; q < V; ++q) o[q] = Elem<T>::from_f(acc[q]);
    *reinterpret_cast<uint4*>(out + (size_t)t * H + c) = res;
  }
}

}  // namespace

hipError_t launch_finalize(const Shape& s, const void* y, const int32_t* inv, const float* w,
                           void* out, hipStream_t st, const void* ys) {
  if (s.bf16)
    hipLaunchKernelGGL(finalize_kernel<uint16_t>, dim3(s.T), dim3(256), 0, st,
                       (const uint16_t*)y, inv, w, (const uint16_t*)ys, s.H, s.k, (uint16_t*)out);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, dim3(s.T), dim3(256), 0, st, (const float*)y, inv,
                       w, (const float*)ys, s.H, s.k, (float*)out);
  return hipGetLastError();
}

}  // namespace moe
