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
// is accumulated on the fp64 matrix pipe, then each wave runs the top-k of
// its tokens with one lane per expert: k rounds of a 64-lane arg-max over the
// key (orderable(logit) << 32 | (63 - e)), so equal logits go to the lower
// expert index.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTokTile = 16;  // tokens per workgroup

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

typedef double f64x4 __attribute__((ext_vector_type(4)));

// 8 consecutive activations of one token as fp32 (exact for bf16 and fp32).
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Logit tile of kTokTile tokens x 64 experts on the fp64 matrix pipe
// (v_mfma_f64_16x16x4_f64, exact products, fp64 sums).  Wave w covers the
// hidden range [w*H/4, (w+1)*H/4) for all four 16-expert tiles; lane
// (t = lane%16, g = lane/16) holds x[t][h0 + 8g + m] and wg[16q + t][h0 + 8g + m]
// as the m-th MFMA's A and B elements, so the 8 MFMAs of a 32-wide chunk sum
// every h of the chunk exactly once.  The four wave partials are added in a
// fixed order, so the logits are reproducible run to run.
template <typename XT>
__global__ __launch_bounds__(256) void route_kernel(const XT* __restrict__ x,
                                                    const float* __restrict__ wg,
                                                    const float* __restrict__ bias, int T, int H,
                                                    int E, int k, float* __restrict__ logits,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ topw) {
  __shared__ double part[4][kTokTile][kMaxExperts + 1];
  __shared__ float lg[kTokTile][kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTokTile;
  const int tl = lane & 15, g = lane >> 4;
  const int hq = H / 4;
  const int hb = wave * hq;

  const bool tok_ok = t0 + tl < T;
  const XT* xrow = x + (size_t)min(t0 + tl, T - 1) * H + hb + 8 * g;
  const float* wrow[4];
  bool w_ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 16 * q + tl;
    w_ok[q] = e < E;
    wrow[q] = wg + (size_t)min(e, E - 1) * H + hb + 8 * g;
  }

  f64x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f64x4{0.0, 0.0, 0.0, 0.0};

  // chunk loads are double-buffered: chunk c+32 is in flight while the
  // 32 MFMAs of chunk c run (hq is a multiple of 64)
  float xv[2][8], wv[2][4][8];
  auto load_chunk = [&](int c, int b) {
    load8(xrow + c, xv[b]);
#pragma unroll
    for (int q = 0; q < 4; ++q) load8(wrow[q] + c, wv[b][q]);
  };
  auto mma_chunk = [&](int b) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const double a = tok_ok ? (double)xv[b][m] : 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, w_ok[q] ? (double)wv[b][q][m] : 0.0, acc[q], 0, 0, 0);
    }
  };
  load_chunk(0, 0);
  for (int c = 0; c < hq; c += 64) {
    load_chunk(c + 32, 1);
    mma_chunk(0);
    if (c + 64 < hq) load_chunk(c + 64, 0);
    mma_chunk(1);
  }
  // fp64 16x16 D layout: register r of lane holds row (lane/16) + 4r (token),
  // column lane%16 (expert)
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][g + 4 * r][16 * q + tl] = acc[q][r];
  __syncthreads();

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx >> 6, e = idx & 63;
    const double s = ((part[0][r][e] + part[1][r][e]) + part[2][r][e]) + part[3][r][e];
    const double b = (bias != nullptr && e < E) ? (double)bias[e] : 0.0;
    const float L = (float)(s + b);
    lg[r][e] = L;
    if (t0 + r < T && e < E) logits[(size_t)(t0 + r) * E + e] = L;
  }
  __syncthreads();

  // top-k: wave w handles tokens w*4 .. w*4+3, lane = expert.
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
