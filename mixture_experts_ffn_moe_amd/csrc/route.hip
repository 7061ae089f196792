// Router logits, top-k selection and renormalised softmax weights.
//
// The router is replicated and runs in fp32 with fp32 weights
// ("HunyuanImage-3.0 on CANN NPU", section 5.2); it yields expert ids and
// routing scores of shape [num_tokens, top_k] ("Hunyuan Image 3.0 hybrid
// parallelism", section 6.1).  Every product x*wg is exact in fp64 (a bf16 or
// fp32 factor times an fp32 factor needs at most 48 significand bits), the
// products are summed in fp64, the bias is added in fp64, and the sum is
// rounded once to fp32.  Any fp64 summation order gives the same fp32 logit
// except within ~1e-16 relative of an fp32 rounding midpoint, which keeps the
// selected experts reproducible against a CPU evaluation.
//
// One workgroup handles kTokTile tokens: the fp64 logit tile [kTokTile x 64]
// is accumulated over H in LDS-staged chunks, then each wave runs the top-k of
// its tokens with one lane per expert: k rounds of a 64-lane arg-max over the
// key (orderable(logit) << 32 | (63 - e)), so equal logits go to the lower
// expert index.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTokTile = 16;  // tokens per workgroup
constexpr int kHChunk = 128;  // hidden elements staged per step
constexpr int kWsPad = 4;     // floats of padding per staged router row

// Orderable 32-bit key of a float: unsigned order equals numeric order and
// -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t orderable(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, d);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  // xor butterfly: every lane adds the same two partial sums (in either
  // order), so all lanes end with the bit-identical total.
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

template <typename XT>
__global__ __launch_bounds__(256) void route_kernel(const XT* __restrict__ x,
                                                    const float* __restrict__ wg,
                                                    const float* __restrict__ bias, int T, int H,
                                                    int E, int k, float* __restrict__ logits,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ topw) {
  __shared__ __attribute__((aligned(16))) float xs[kTokTile][kHChunk];
  __shared__ __attribute__((aligned(16))) float ws[kMaxExperts][kHChunk + kWsPad];
  __shared__ float lg[kTokTile][kMaxExperts];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTokTile;
  const int e = tid & 63;          // expert of this thread's logits
  const int tg = tid >> 6;         // token group: tokens tg*4 .. tg*4+3

  double acc[4] = {0.0, 0.0, 0.0, 0.0};

  for (int h0 = 0; h0 < H; h0 += kHChunk) {
    // x chunk: 16 tokens x 128 values, 8 consecutive values per thread.
    {
      const int idx = tid * 8;
      const int r = idx / kHChunk, c = idx % kHChunk;
      const int t = t0 + r;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        xs[r][c + q] = (t < T) ? Elem<XT>::to_f(x[(size_t)t * H + h0 + c + q]) : 0.0f;
    }
    // router chunk: 64 experts x 128 values, 8 float4 per thread.
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = (tid + q * 256) * 4;
      const int r = idx / kHChunk, c = idx % kHChunk;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < E) v = *reinterpret_cast<const float4*>(wg + (size_t)r * H + h0 + c);
      *reinterpret_cast<float4*>(&ws[r][c]) = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kHChunk; c += 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(&ws[e][c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x4 = *reinterpret_cast<const float4*>(&xs[tg * 4 + i][c]);
        acc[i] = fma((double)x4.x, (double)w4.x, acc[i]);
        acc[i] = fma((double)x4.y, (double)w4.y, acc[i]);
        acc[i] = fma((double)x4.z, (double)w4.z, acc[i]);
        acc[i] = fma((double)x4.w, (double)w4.w, acc[i]);
      }
    }
    __syncthreads();
  }

  const double b = (bias != nullptr && e < E) ? (double)bias[e] : 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tg * 4 + i, t = t0 + r;
    const float L = (float)(acc[i] + b);
    lg[r][e] = L;
    if (t < T && e < E) logits[(size_t)t * E + e] = L;
  }
  __syncthreads();

  // top-k: wave w handles tokens w*4 .. w*4+3, lane = expert.
  const int wave = tid >> 6, lane = tid & 63;
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 4 + i, t = t0 + r;
    if (t >= T) break;
    uint64_t key = 0;
    if (lane < E) key = ((uint64_t)orderable(lg[r][lane]) << 32) | (uint32_t)(63 - lane);
    float mine = 0.0f;    // lane j keeps the j-th selected logit
    float first = 0.0f;   // the largest logit
    for (int j = 0; j < k; ++j) {
      const uint64_t m = wave_max_u64(key);
      const int win = 63 - (int)(m & 0xffffffffu);
      const float Lw = from_orderable((uint32_t)(m >> 32));
      if (j == 0) first = Lw;
      if (lane == j) mine = Lw;
      if (lane == win) key = 0;
      if (lane == 0) ids[(size_t)t * k + j] = win;
    }
    // weights: softmax restricted to the selected experts (the full softmax
    // denominator cancels in the renormalisation), in fp64.
    const double ex = (lane < k) ? exp((double)mine - (double)first) : 0.0;
    const double s = wave_sum_f64(ex);
    if (lane < k) topw[(size_t)t * k + lane] = (float)(ex / s);
  }
}

}  // namespace

hipError_t launch_route(const Shape& s, const void* x, const float* wg, const float* bias,
                        float* logits, int32_t* ids, float* w, hipStream_t st) {
  const int blocks = (s.T + kTokTile - 1) / kTokTile;
  if (s.bf16)
    hipLaunchKernelGGL(route_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st,
                       (const uint16_t*)x, wg, bias, s.T, s.H, s.E, s.k, logits, ids, w);
  else
    hipLaunchKernelGGL(route_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)x, wg,
                       bias, s.T, s.H, s.E, s.k, logits, ids, w);
  return hipGetLastError();
}

}  // namespace moe
