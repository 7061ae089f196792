// Router logits, top-k selection and softmax weights (renormalised over the
// selected experts, or not).
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
// its tokens with one lane per expert: k rounds of a 64-lane maximum of the
// orderable logit key, the winner being the lowest lane that holds it, so
// equal logits go to the lower expert index.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTokTile = kRouteTokTile;  // tokens per workgroup

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
// (v_mfma_f64_16x16x4_f64, exact products, fp64 sums).  Sixteen waves, four
// per SIMD (one wave alone cannot keep the matrix pipe busy, and four hide the
// activation loads from HBM better than two): wave w covers the hidden part
// w -- the 32-wide chunks [w*nc/16, (w+1)*nc/16) of the nc = H/32 chunks, a
// sixteenth of H when H % 512 == 0 -- for all four 16-expert tiles q, so each
// activation is loaded and converted once per workgroup (with a quarter of the
// experts per wave it was loaded twice: 2-3 % slower); lane (t = lane%16,
// g = lane/16) holds x[t][h0 + 8g + m] and wg[16q + t][h0 + 8g + m] as the
// m-th MFMA's A and B elements, so the 8 MFMAs of a 32-wide chunk and tile sum
// every h of the chunk exactly once.  The sixteen partials are added in a
// fixed order, so the logits are reproducible run to run.
constexpr int kRouteWaves = 16;
constexpr int kHParts = kRouteWaves;  // hidden parts (each wave: one part, all 64 experts)

template <typename XT>
__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(const XT* __restrict__ x,
                                                    const float* __restrict__ wg,
                                                    const float* __restrict__ bias, int T, int H,
                                                    int E, int k, float* __restrict__ logits,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ topw,
                                                    int32_t* __restrict__ hist, int renorm) {
  __shared__ double part[kHParts][kTokTile][kMaxExperts + 1];
  __shared__ float lg[kTokTile][kMaxExperts];
  __shared__ int hcnt[kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hw = wave;  // hidden part
  const int t0 = blockIdx.x * kTokTile;
  const int tl = lane & 15, g = lane >> 4;
  const int nc = H / 32;  // 32-wide chunks of the hidden dimension
  const int cb = hw * nc / kHParts, ce = (hw + 1) * nc / kHParts;
  const int hb = cb * 32, hq = (ce - cb) * 32;  // this part's first column and width (hq may be 0)

  if (tid < kMaxExperts) hcnt[tid] = 0;  // ordered before its use by the barriers below

  // rows past T and experts past E read the last valid row instead: their
  // logits are computed but never stored or ranked, so no operand is masked
  const XT* xrow = x + (size_t)min(t0 + tl, T - 1) * H + hb + 8 * g;
  const float* wrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 16 * q + tl;
    wrow[q] = wg + (size_t)min(e, E - 1) * H + hb + 8 * g;
  }

  f64x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f64x4{0.0, 0.0, 0.0, 0.0};

  // one chunk in registers at a time (hq is a multiple of 32, possibly 0):
  // four waves per SIMD overlap one wave's loads with the others' MFMAs (a
  // second chunk in flight per wave would spill at four expert tiles)
  float xv[8], wv[4][8];
  for (int c = 0; c < hq; c += 32) {
    load8(xrow + c, xv);
#pragma unroll
    for (int q = 0; q < 4; ++q) load8(wrow[q] + c, wv[q]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const double a = (double)xv[m];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)wv[q][m], acc[q], 0, 0, 0);
    }
  }
  // fp64 16x16 D layout: register r of lane holds row (lane/16) + 4r (token),
  // column lane%16 (expert)
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[hw][g + 4 * r][16 * q + tl] = acc[q][r];
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kTokTile * kMaxExperts / (kRouteWaves * 64); ++i) {
    const int idx = tid + kRouteWaves * 64 * i;
    const int r = idx >> 6, e = idx & 63;
    double s = part[0][r][e];
#pragma unroll
    for (int p = 1; p < kHParts; ++p) s += part[p][r][e];
    const double b = (bias != nullptr && e < E) ? (double)bias[e] : 0.0;
    const float L = (float)(s + b);
    lg[r][e] = L;
    if (t0 + r < T && e < E) logits[(size_t)(t0 + r) * E + e] = L;
  }
  __syncthreads();

  // top-k: wave w handles tokens w*2 and w*2+1, lane = expert.
  constexpr int kTokPerWave = kTokTile / kRouteWaves;
  for (int i = 0; i < kTokPerWave; ++i) {
    const int r = wave * kTokPerWave + i, t = t0 + r;
    if (t >= T) break;
    // key 0 is below every finite logit's key: it marks lanes past E and
    // experts already taken
    uint32_t key = lane < E ? orderable(lg[r][lane]) : 0u;
    float mine = 0.0f;    // lane j keeps the j-th selected logit
    float first = 0.0f;   // the largest logit
    for (int j = 0; j < k; ++j) {
      const uint32_t m = wave_max_u32(key);
      // the lowest lane holding the maximum: equal logits go to the lower expert
      const int win = __ffsll((long long)__ballot(key == m)) - 1;
      const float Lw = from_orderable(m);
      if (j == 0) first = Lw;
      if (lane == j) mine = Lw;
      if (lane == win) key = 0;
      if (lane == 0) {
        ids[(size_t)t * k + j] = win;
        if (hist != nullptr) atomicAdd(&hcnt[win], 1);
      }
    }
    // weights in fp64: renormalised, the softmax restricted to the selected
    // experts (the full softmax denominator cancels); else the softmax over
    // all E experts at the selected ones
    const double ex = (lane < k) ? exp((double)mine - (double)first) : 0.0;
    const double s = wave_sum_f64(renorm ? ex : (lane < E ? exp((double)lg[r][lane] - (double)first) : 0.0));
    if (lane < k) topw[(size_t)t * k + lane] = (float)(ex / s);
  }
  if (hist != nullptr) {
    __syncthreads();
    if (tid < kMaxExperts) hist[(size_t)blockIdx.x * kMaxExperts + tid] = hcnt[tid];
  }
}

}  // namespace

hipError_t launch_route(const Shape& s, const void* x, const float* wg, const float* bias,
                        float* logits, int32_t* ids, float* w, hipStream_t st, int32_t* hist) {
  const int blocks = (s.T + kTokTile - 1) / kTokTile;
  const dim3 block(kRouteWaves * 64);
  if (s.bf16)
    hipLaunchKernelGGL(route_kernel<uint16_t>, dim3(blocks), block, 0, st,
                       (const uint16_t*)x, wg, bias, s.T, s.H, s.E, s.k, logits, ids, w, hist,
                       (int)s.renorm);
  else
    hipLaunchKernelGGL(route_kernel<float>, dim3(blocks), block, 0, st, (const float*)x, wg,
                       bias, s.T, s.H, s.E, s.k, logits, ids, w, hist, (int)s.renorm);
  return hipGetLastError();
}

}  // namespace moe
