// Expert counts, exclusive offsets and the stable route permutation.
//
// "Hunyuan Image 3.0 hybrid parallelism", section 6.1: the flattened expert
// ids are sorted by expert into permuted_to_expanded, bincount + cumsum give
// the per-expert offsets, and finalize reads routes back through the inverse
// permutation.  The sort here is a counting sort, stable in the route index
// r = t*k + j, so each expert's rows stay in token order and the result is
// unique (bit-exact against any other stable sort).
//
// One workgroup of 16 waves.  Wave w owns the contiguous route chunk
// [w*C, (w+1)*C).  Pass 1 counts experts per wave; one wave then turns the
// [16 x E] counts into offsets and per-(wave, expert) write bases; pass 2
// walks each chunk 64 routes at a time, ranks every route among the earlier
// lanes with the same expert (six ballots over the id bits), and scatters.
// Counts use LDS atomics (order-independent); positions use none, so perm and
// inv are deterministic.  The routes are at most T*k = 64K here, so one CU
// finishes in a few microseconds and no grid-wide synchronisation is needed.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kWaves = 16;

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ ids, int R,
                                                       int E, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv) {
  __shared__ int cnt[kWaves][kMaxExperts];
  __shared__ int base[kWaves][kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  const int per = (R + kWaves - 1) / kWaves;
  const int C = (per + 63) & ~63;
  const int start = min(R, wave * C), end = min(R, start + C);

  cnt[wave][lane] = 0;
  __syncthreads();
  for (int r = start + lane; r < end; r += kWave) {
    int v = ids[r];
    v = min(max(v, 0), E - 1);  // ids come from the router; clamp keeps writes in bounds
    atomicAdd(&cnt[wave][v], 1);
  }
  __syncthreads();

  if (wave == 0) {
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = (lane < E) ? cnt[w][lane] : 0;
      base[w][lane] = tot;
      tot += c;
    }
    int incl = tot;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int excl = incl - tot;
    for (int w = 0; w < kWaves; ++w) base[w][lane] += excl;
    if (lane < E) {
      counts[lane] = tot;
      offsets[lane] = excl;
    }
    if (lane == E - 1) offsets[E] = incl;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int r0 = start; r0 < end; r0 += kWave) {
    const int r = r0 + lane;
    const bool valid = r < end;
    int v = valid ? ids[r] : 0;
    v = min(max(v, 0), E - 1);
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const bool bit = (v >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    int rank = 0, pos = 0;
    if (valid) {
      rank = __popcll(peers & lt_mask);
      pos = base[wave][v] + rank;
      perm[pos] = r;
      inv[r] = pos;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) base[wave][v] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x,
                                                     const int32_t* __restrict__ perm, int H,
                                                     int k, T* __restrict__ xp) {
  const int p = blockIdx.x;
  const int t = perm[p] / k;
  constexpr int V = 16 / sizeof(T);
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  uint4* dst = reinterpret_cast<uint4*>(xp + (size_t)p * H);
  for (int c = threadIdx.x; c < H / V; c += blockDim.x) dst[c] = src[c];
}

}  // namespace

hipError_t launch_permute(const Shape& s, const int32_t* ids, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t st) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kWaves * kWave), 0, st, ids, (int)s.R(), s.E,
                     counts, offsets, perm, inv);
  return hipGetLastError();
}

hipError_t launch_gather(const Shape& s, const void* x, const int32_t* perm, void* xp,
                         hipStream_t st) {
  const unsigned R = (unsigned)s.R();
  if (s.bf16)
    hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3(R), dim3(256), 0, st, (const uint16_t*)x,
                       perm, s.H, s.k, (uint16_t*)xp);
  else
    hipLaunchKernelGGL(gather_kernel<float>, dim3(R), dim3(256), 0, st, (const float*)x, perm,
                       s.H, s.k, (float*)xp);
  return hipGetLastError();
}

}  // namespace moe
