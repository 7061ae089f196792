// Small-token (AR decode) path of the routed MoE layer.
//
// In the AR phase each rank runs the MoE for a handful of tokens on its
// micro view of the resident shard ("Hunyuan Image 3.0 hybrid parallelism",
// sections 4.3 and 6.2).  With T <= 16 tokens every expert sees at most T
// rows, so the layer is a stream over the active experts' weights: the time
// is the HBM time of those weights, and the job of these kernels is to keep
// enough bytes in flight and to spend no extra launches or passes.
//
//   1. decode_route_partial: fp64 router partial sums, the hidden dimension
//      split over kSplit workgroups (one CU could not stream the router
//      weights fast enough), exact products on v_mfma_f64_16x16x4_f64; each
//      of a workgroup's 16 waves takes a hidden quarter and 16 experts, so
//      four waves share a SIMD's matrix pipe (one wave alone keeps it half
//      busy).
//   2. routing finish, at the start of every decode_w13 workgroup (cheaper
//      than a launch of its own): fixed-order sum of the partials, bias, one
//      fp32 rounding, top-k and weights (same rules as route.hip), expert
//      counts and offsets, the stable permutation and its inverse, and the
//      ascending list of active experts; workgroup 0 writes them out.
//   3. decode_w13: one wave per (active expert, 8 columns of the micro-major
//      intermediate), the waves' units dealt evenly over one workgroup per
//      CU; each wave streams its 8 gate and 8 up rows of w1 straight to LDS in
//      512-byte runs, reads them back as one MFMA B fragment (M = the
//      expert's rows, padded to 16) and applies SwiGLU; h is rounded to bf16.
//   4. decode_down_finalize: one workgroup per 16 output columns; its 16
//      waves split the active experts (enough loads in flight per CU), stream
//      the matching w2 rows the same way, and put
//      w[t, j] * y[route (t, j)] into a per-route LDS slot; the slots are then
//      summed in ascending j (the finalize of section 6.1), so the down
//      partials of every micro-shard and route are reduced once, without
//      atomics and without a y tensor.
// With a shared expert ("HunyuanImage-3.0 on CANN NPU", section 3.1) its
// weights stream in the same two launches: decode_w13 runs its gate|up
// columns for every token as extra units of its work list, and
// decode_down_finalize takes it as one more work item whose per-token slot
// (weight 1) is added after the routed sum.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kDecT = 16;       // token tile (max tokens on this path)
constexpr int kSplit = 16;      // router split of the hidden dimension
constexpr int kMaxK = 64;

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

__device__ __forceinline__ void load8f(const uint16_t* p, float (&v)[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// ---------------------------------------------------------------------------
// 1. router partials: block s covers hidden [s*H/kSplit, (s+1)*H/kSplit), its
// wave w the quarter w % 4 of that for experts [16*(w/4), 16*(w/4) + 16);
// partial[s][t][e] (fp64, the quarters summed in a fixed order).
constexpr int kRouteWaves = 16;
__global__ __launch_bounds__(kRouteWaves * 64) void decode_route_partial(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wg, int T,
                                                            int H, int E,
                                                            double* __restrict__ partial) {
  __shared__ double part[4][kDecT][kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tl = lane & 15, g = lane >> 4;
  const int hw = wave & 3, q = wave >> 2;  // hidden quarter, expert tile
  const int hs = H / kSplit, hq = hs / 4;
  const int hb = blockIdx.x * hs + hw * hq;
  // tokens past T and experts past E read the last valid row: their partials
  // are never used, so no operand is masked
  const uint16_t* xrow = x + (size_t)min(tl, T - 1) * H + hb + 8 * g;
  const float* wrow = wg + (size_t)min(16 * q + tl, E - 1) * H + hb + 8 * g;
  f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
  float xv[2][8], wv[2][8];
  auto load_chunk = [&](int c, int b) {
    load8f(xrow + c, xv[b]);
    const float4 a = *reinterpret_cast<const float4*>(wrow + c);
    const float4 bb = *reinterpret_cast<const float4*>(wrow + c + 4);
    wv[b][0] = a.x; wv[b][1] = a.y; wv[b][2] = a.z; wv[b][3] = a.w;
    wv[b][4] = bb.x; wv[b][5] = bb.y; wv[b][6] = bb.z; wv[b][7] = bb.w;
  };
  auto mma_chunk = [&](int b) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[b][m], (double)wv[b][m], acc, 0, 0, 0);
  };
  // hq = H / 64 is a multiple of 32: pairs of chunks (the second in flight
  // while the first is consumed), then one trailing chunk when hq % 64 == 32
  int c = 0;
  for (; c + 64 <= hq; c += 64) {
    load_chunk(c, 0);
    load_chunk(c + 32, 1);
    mma_chunk(0);
    mma_chunk(1);
  }
  if (c < hq) {
    load_chunk(c, 0);
    mma_chunk(0);
  }
  // fp64 16x16 D layout: register r holds row (lane/16) + 4r, column lane%16
#pragma unroll
  for (int r = 0; r < 4; ++r) part[hw][g + 4 * r][16 * q + tl] = acc[r];
  __syncthreads();
  {
    const int r = tid >> 6, e = tid & 63;
    partial[((size_t)blockIdx.x * kDecT + r) * kMaxExperts + e] =
        ((part[0][r][e] + part[1][r][e]) + part[2][r][e]) + part[3][r][e];
  }
}

// ---------------------------------------------------------------------------
// 2. routing of the token tile, run by one workgroup of 16 waves (each
// workgroup of decode_w13 runs it for itself at its start: the inputs are the
// router partials, 128 KB in L2, and the work is a few microseconds, less
// than a separate launch and kernel boundary).  Workgroup `out` writes the
// routing outputs to memory; every workgroup keeps the offsets, the active
// experts and the permutation in LDS for its own use.
struct RouteLds {
  float lg[kDecT][kMaxExperts];
  int sids[kDecT * kMaxK];
  uint64_t sel[kDecT];           // experts chosen by each token
  int base[kMaxExperts];
  int off[kMaxExperts + 1];      // expert offsets
  int act[kMaxExperts + 1];      // active experts ascending; their number in act[kMaxExperts]
  int perm[kDecT * kMaxK];       // permuted row -> route
};

__device__ __forceinline__ void route_finish(
    const double* __restrict__ partial, const float* __restrict__ bias, int T, int E, int k, bool renorm,
    bool out, float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ topw,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ active, RouteLds& S) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  {  // logits: thread (r, e), partials summed in split order (rows past T
     // are never ranked: their partials are not read)
    const int r = tid >> 6, e = tid & 63;
    double s = 0.0;
    if (r < T)
      for (int b = 0; b < kSplit; ++b) s += partial[((size_t)b * kDecT + r) * kMaxExperts + e];
    const double bb = (bias != nullptr && e < E) ? (double)bias[e] : 0.0;
    const float L = (float)(s + bb);
    S.lg[r][e] = L;
    if (out && r < T && e < E) logits[(size_t)r * E + e] = L;
  }
  __syncthreads();

  {  // top-k and weights: wave = token, lane = expert (same rules as route.hip)
    const int t = wave;
    if (t < T) {
      uint32_t key = lane < E ? orderable(S.lg[t][lane]) : 0u;
      bool taken = false;
      float mine = 0.0f, first = 0.0f;
      for (int j = 0; j < k; ++j) {
        const uint32_t m = wave_max_u32(key);
        const int win = __ffsll((long long)__ballot(key == m)) - 1;
        const float Lw = from_orderable(m);
        if (j == 0) first = Lw;
        if (lane == j) mine = Lw;
        if (lane == win) {
          key = 0;
          taken = true;
        }
        if (lane == 0) {
          if (out) ids[(size_t)t * k + j] = win;
          S.sids[t * k + j] = win;
        }
      }
      const uint64_t chosen = __ballot(taken);
      if (lane == 0) S.sel[t] = chosen;
      const double ex = (lane < k) ? exp((double)mine - (double)first) : 0.0;
      const double s =
          wave_sum_f64(renorm ? ex : (lane < E ? exp((double)S.lg[t][lane] - (double)first) : 0.0));
      if (out && lane < k) topw[(size_t)t * k + lane] = (float)(ex / s);
    }
  }
  __syncthreads();

  // counts, offsets, active list (wave 0, lane = expert): a token chooses an
  // expert at most once, so the count is the number of tokens whose
  // selection holds it
  const int R = T * k;
  if (wave == 0) {
    int c = 0;
    for (int t = 0; t < T; ++t) c += (int)((S.sel[t] >> lane) & 1ull);
    int incl = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int excl = incl - c;
    S.base[lane] = excl;
    if (lane < E) {
      S.off[lane] = excl;
      if (out) {
        counts[lane] = c;
        offsets[lane] = excl;
      }
    }
    if (lane == E - 1) {
      S.off[E] = incl;
      if (out) offsets[E] = incl;
    }
    // active experts in ascending order: position = number of active experts below
    const uint64_t act = __ballot(lane < E && c > 0);
    const uint64_t below = (lane == 0) ? 0ull : (act & ((~0ull) >> (64 - lane)));
    if (lane < E && c > 0) {
      S.act[__popcll(below)] = lane;
      if (out) active[__popcll(below)] = lane;
    }
    if (lane == 0) {
      S.act[kMaxExperts] = __popcll(act);
      if (out) active[kMaxExperts] = __popcll(act);
    }
  }
  __syncthreads();
  // stable scatter: the routes of expert e before r = t*k + j are those of
  // the earlier tokens that chose e
  for (int r = tid; r < R; r += blockDim.x) {
    const int t = r / k, e = S.sids[r];
    int rank = 0;
    for (int q = 0; q < t; ++q) rank += (int)((S.sel[q] >> e) & 1ull);
    const int p = S.base[e] + rank;
    S.perm[p] = r;
    if (out) {
      perm[p] = r;
      inv[r] = p;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Weight streaming of the down projection.  A wave reads 16 weight rows per
// 64-element k-step as two loads of 8 rows x 128 bytes (eight lanes per row:
// every load covers whole 128-byte lines, which HBM serves markedly faster
// than the 64-byte halves the MFMA fragment layout would ask for), writes them
// to a per-wave LDS buffer and reads them back in the 16x16x32 B-fragment
// layout (lane l: row l % 16, 8 consecutive k of chunk l / 16).  Within a
// 128-byte row the 16-byte chunks are XOR-swizzled by (row / 2) % 8, so the 16
// lanes of one LDS phase hit 16 bank groups on both sides.  The k order inside
// each MFMA is the one the grouped GEMMs use.
constexpr int kStep = 64;        // k per LDS round trip
constexpr int kStepsDown = 4;    // the same for the down projection
constexpr int kDownWaves = 16;   // waves of the down+finalize workgroup (they split the experts)

struct WaveRows {
  // byte offsets of this lane in a 16-row x 128-byte block: its load slot and
  // its fragment-read slot for the two 32-element halves of a k-step
  uint32_t wr0, wr1, rd0, rd1;
  __device__ __forceinline__ explicit WaveRows(int lane) {
    const int r0 = lane >> 3, r1 = 8 + (lane >> 3), c = lane & 7;
    wr0 = (uint32_t)(r0 * 128 + ((c ^ ((r0 >> 1) & 7)) * 16));
    wr1 = (uint32_t)(r1 * 128 + ((c ^ ((r1 >> 1) & 7)) * 16));
    const int fr = lane & 15, g = lane >> 4;
    rd0 = (uint32_t)(fr * 128 + (((0 + g) ^ ((fr >> 1) & 7)) * 16));
    rd1 = (uint32_t)(fr * 128 + (((4 + g) ^ ((fr >> 1) & 7)) * 16));
  }
};

// ---------------------------------------------------------------------------
// 3. gate|up + SwiGLU.  The work is a list of units, one per (active expert,
// 8 intermediate columns) and then one per 8 columns of the shared expert; a
// unit is one wave's stream of its 8 gate and 8 up rows over all of H, the
// 16 rows of one MFMA B fragment (output columns 0-7 gate, 8-15 up).  Each of
// the kW13Blocks workgroups takes an equal contiguous share of the list (the
// list length is known only on the device), its waves taking the share's
// units in turn: every CU streams the same number of bytes to within one
// 128 KB unit, whatever the number of active experts.  (A unit of 16 gate and
// 16 up rows left half the waves idle at 42 active experts and, with the
// shared expert's units added, put a ninth 256 KB unit on some CUs: +12 %.)
//
// The rows go straight to a per-wave LDS slot by direct-to-LDS copies, each
// copy 2 rows x 512 contiguous bytes; a row's 16-byte chunk c sits at slot
// position c ^ (row % 16), so the fragment reads (16 rows, one chunk column)
// hit 16 bank groups.  Each MFMA takes the 32 k of one chunk column in the
// same lane order as the grouped GEMMs, in ascending k: h is the same bits on
// both paths.
constexpr int kW13Waves = 16;    // waves per workgroup; a wave takes every 16th unit of its share
constexpr int kW13Blocks = 256;  // one workgroup per CU
constexpr int kSeg = 256;        // k per slot fill: 512 contiguous bytes of every row of the unit
constexpr int kUnitCols = 8;     // gate (and up) rows per unit

__global__ __launch_bounds__(kW13Waves * 64) void decode_w13(
    const uint16_t* __restrict__ x, const double* __restrict__ partial, const float* __restrict__ bias,
    const uint16_t* __restrict__ w1, int T, int H, int E, int k, int Im, int mu,
    uint16_t* __restrict__ h, const uint16_t* __restrict__ w1s, int Is, uint16_t* __restrict__ hs,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ topw,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets_out, int32_t* __restrict__ perm_out,
    int32_t* __restrict__ inv, int32_t* __restrict__ active_out, int renorm) {
  static_assert(kW13Waves * 64 == kDecT * kMaxExperts, "routing: one thread per (token, expert)");
  constexpr int kSlot = 2 * kUnitCols * kSeg * 2;  // bytes: 16 rows x 512
  __shared__ __attribute__((aligned(1024))) char buf[kW13Waves][kSlot];
  __shared__ RouteLds rs;
  route_finish(partial, bias, T, E, k, renorm != 0, blockIdx.x == 0, logits, ids, topw, counts, offsets_out, perm_out,
               inv, active_out, rs);
  const int* active = rs.act;
  const int* offsets = rs.off;
  const int* perm = rs.perm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, g4 = lane >> 4;
  const int ue = mu * Im / kUnitCols;  // units per routed expert
  const int routed_units = active[kMaxExperts] * ue;
  const int units = routed_units + (w1s != nullptr ? Is / kUnitCols : 0);
  const int u_end = (int)((long long)(blockIdx.x + 1) * units / gridDim.x);
  const uint32_t slot = (uint32_t)(uintptr_t)buf[wave];
  // copy q of a fill: unit row 2q + lane/32, slot position lane % 32 holding
  // the row's chunk (lane % 32) ^ (row % 16)
  const int crow = lane >> 5, cpos = lane & 31;
  for (int u = (int)((long long)blockIdx.x * units / gridDim.x) + wave; u < u_end; u += kW13Waves) {
    int n, c0, i0, Imx, ldh;
    const uint16_t* arow;
    const uint16_t* wbase;
    uint16_t* hout;
    if (u >= routed_units) {
      // shared expert: every token, in order
      n = T;
      c0 = (u - routed_units) * kUnitCols;
      i0 = c0;
      Imx = Is;
      ldh = Is;
      arow = x + (size_t)min(fr, n - 1) * H + g4 * 8;
      wbase = w1s;
      hout = hs;
    } else {
      const int e = active[u / ue];
      const int seg = offsets[e];
      n = offsets[e + 1] - seg;
      c0 = (u % ue) * kUnitCols;  // column in [0, mu*Im)
      const int micro = c0 / Im;
      i0 = c0 - micro * Im;
      Imx = Im;
      ldh = mu * Im;
      // rows past the expert's repeat its last token (finite values in MFMA
      // rows that are never stored)
      arow = x + (size_t)(perm[seg + min(fr, n - 1)] / k) * H + g4 * 8;
      wbase = w1 + (size_t)(micro * E + e) * 2 * Im * H;
      hout = h + (size_t)seg * ldh;
    }
    // unit row r < 8: gate row i0 + r; r >= 8: up row Imx + i0 + r - 8
    const uint16_t* sb = uniform_ptr(wbase + (size_t)i0 * H);
    uint32_t voff[kUnitCols];
#pragma unroll
    for (int q = 0; q < kUnitCols; ++q) {
      const int r = 2 * q + crow;
      const int wr = r < kUnitCols ? r : Imx + r - kUnitCols;
      voff[q] = ((uint32_t)wr * (uint32_t)H + (uint32_t)((cpos ^ (r & 15)) * 8)) * 2u;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < H; k0 += kSeg) {
      // the fragment reads of the previous fill are done before the slot is refilled
      __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < kUnitCols; ++q) dma16(slot + q * 1024u, sb + k0, voff[q]);
      uint4 av[kSeg / 32];
#pragma unroll
      for (int j = 0; j < kSeg / 32; ++j) av[j] = *reinterpret_cast<const uint4*>(arow + k0 + 32 * j);
      wait_vmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kSeg / 32; ++j) {
        const uint4 b = *reinterpret_cast<const uint4*>(buf[wave] + fr * (kSeg * 2) + (((4 * j + g4) ^ fr) * 16));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[j]), __builtin_bit_cast(bf16x8, b),
                                                      acc, 0, 0, 0);
      }
    }
    // D layout: register r holds row 4*(lane/16) + r, column lane%16 (gate
    // columns 0-7, their up columns 8-15)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float up = __shfl_xor(acc[r], 8);
      const int row = 4 * g4 + r;
      if (fr < kUnitCols && row < n)
        hout[(size_t)row * ldh + c0 + fr] = float_to_bf16_bits(silu_f32(acc[r]) * up);
    }
  }  // units of this wave
}

// ---------------------------------------------------------------------------
// 4. down projection + finalize for 16 output columns and all tokens.
__global__ __launch_bounds__(kDownWaves * 64) void decode_down_finalize(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const float* __restrict__ topw, const uint16_t* __restrict__ w2, int T, int H, int E, int k,
    int Im, int mu, uint16_t* __restrict__ out, const uint16_t* __restrict__ hs,
    const uint16_t* __restrict__ w2s, int Is) {
  __shared__ float slot[kDecT * kMaxK][16];
  __shared__ float sslot[kDecT][16];  // the shared expert's output, per token
  __shared__ __attribute__((aligned(16))) char buf[kDownWaves][2048];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const int n_act = active[kMaxExperts];
  const bool has_shared = hs != nullptr;
  const int n_items = n_act + (has_shared ? 1 : 0);  // item n_act is the shared expert
  const WaveRows wr(lane);
  char* wb = buf[wave];

  for (int a = wave; a < n_items; a += kDownWaves) {
    const bool sh = a == n_act;
    int n, K, Imx, seg = 0;
    size_t mstride;
    const uint16_t* arow;
    const uint16_t* b0;
    // rows n0 + lane/8 and n0 + 8 + lane/8 of the down weights, chunk lane % 8
    if (sh) {
      n = T;
      K = Is;
      Imx = Is;
      mstride = 0;
      arow = hs + (size_t)min(fr, n - 1) * Is + fk;
      b0 = w2s + (size_t)(n0 + (lane >> 3)) * Is + (lane & 7) * 8;
    } else {
      const int e = active[a];
      seg = offsets[e];
      n = offsets[e + 1] - seg;
      K = mu * Im;
      Imx = Im;
      mstride = (size_t)E * H * Im;
      arow = h + (size_t)(seg + min(fr, n - 1)) * K + fk;
      b0 = w2 + ((size_t)e * H + n0 + (lane >> 3)) * Im + (lane & 7) * 8;
    }
    const bool row_ok = fr < n;
    const size_t r8 = (size_t)8 * Imx;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += kStep * kStepsDown) {
      uint4 bv[kStepsDown][2], av[kStepsDown][2];
#pragma unroll
      for (int q = 0; q < kStepsDown; ++q) {
        const int kg = k0 + kStep * q;  // a 64-step never crosses a micro boundary (Im % 256 == 0)
        const int mm = kg / Imx;
        const uint16_t* bp = b0 + (size_t)mm * mstride + (kg - mm * Imx);
        bv[q][0] = *reinterpret_cast<const uint4*>(bp);
        bv[q][1] = *reinterpret_cast<const uint4*>(bp + r8);
        av[q][0] = row_ok ? *reinterpret_cast<const uint4*>(arow + kg) : make_uint4(0, 0, 0, 0);
        av[q][1] = row_ok ? *reinterpret_cast<const uint4*>(arow + kg + 32) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < kStepsDown; ++q) {
        *reinterpret_cast<uint4*>(wb + wr.wr0) = bv[q][0];
        *reinterpret_cast<uint4*>(wb + wr.wr1) = bv[q][1];
        const uint4 f0 = *reinterpret_cast<const uint4*>(wb + wr.rd0);
        const uint4 f1 = *reinterpret_cast<const uint4*>(wb + wr.rd1);
        uint4 a0 = av[q][0], a1 = av[q][1];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                      __builtin_bit_cast(bf16x8, f0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                      __builtin_bit_cast(bf16x8, f1), acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * (lane >> 4) + r;
      if (row < n) {
        if (sh) {
          sslot[row][fr] = acc[r];
        } else {
          const int route = perm[seg + row];  // = t * k + j
          slot[route][fr] = topw[route] * acc[r];
        }
      }
    }
  }
  __syncthreads();
  // out[t, n0 + c] = sum over j ascending of the route slots, then the shared
  // expert's slot
  for (int i = threadIdx.x; i < T * 16; i += blockDim.x) {
    const int t = i >> 4, c = i & 15;
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s += slot[t * k + j][c];
    if (has_shared) s += sslot[t][c];
    out[(size_t)t * H + n0 + c] = float_to_bf16_bits(s);
  }
}

}  // namespace

size_t decode_scratch_bytes() {
  return (size_t)kSplit * kDecT * kMaxExperts * sizeof(double) + (kMaxExperts + 1) * sizeof(int32_t);
}

bool decode_shared_supported(int Is) {
  return Is > 0 && (Is % 64) == 0 && (Is % (kStep * kStepsDown)) == 0;
}

bool decode_supported(const Shape& s) {
  return s.bf16 && s.T >= 1 && s.T <= kDecT && s.k <= kMaxK && (s.H % (kSplit * 128)) == 0 &&
         (s.Im % 64) == 0 && (s.mu * s.Im) % 64 == 0 && (s.H % kSeg) == 0 &&
         (s.Im % (kStep * kStepsDown)) == 0 && (s.H % 16) == 0;
}

hipError_t launch_decode(const Shape& s, const void* x, const float* wg, const float* bias,
                         const void* w1, const void* w2, void* out, float* logits, int32_t* ids,
                         float* w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                         void* h, void* scratch, hipStream_t st, const SharedExpert* shared) {
  double* partial = (double*)scratch;
  int32_t* active = (int32_t*)((char*)scratch + (size_t)kSplit * kDecT * kMaxExperts * sizeof(double));
  hipLaunchKernelGGL(decode_route_partial, dim3(kSplit), dim3(kRouteWaves * 64), 0, st, (const uint16_t*)x, wg,
                     s.T, s.H, s.E, partial);
  const uint16_t* w1s = shared ? (const uint16_t*)shared->w1 : nullptr;
  const uint16_t* w2s = shared ? (const uint16_t*)shared->w2 : nullptr;
  uint16_t* hs = shared ? (uint16_t*)shared->h : nullptr;
  const int Is = shared ? shared->Is : 0;
  hipLaunchKernelGGL(decode_w13, dim3(kW13Blocks), dim3(kW13Waves * 64), 0, st, (const uint16_t*)x,
                     partial, bias, (const uint16_t*)w1, s.T, s.H, s.E, s.k, s.Im, s.mu, (uint16_t*)h,
                     w1s, Is, hs, logits, ids, w, counts, offsets, perm, inv, active, (int)s.renorm);
  hipLaunchKernelGGL(decode_down_finalize, dim3(s.H / 16), dim3(kDownWaves * 64), 0, st, (const uint16_t*)h,
                     perm, offsets, active, w, (const uint16_t*)w2, s.T, s.H, s.E, s.k, s.Im,
                     s.mu, (uint16_t*)out, (const uint16_t*)hs, w2s, Is);
  return hipGetLastError();
}

}  // namespace moe
