// Grouped expert GEMMs over variable-length expert segments.
//
// "Hunyuan Image 3.0 hybrid parallelism", section 6.1: every micro-shard runs
// grouped GEMM1 (fused gate|up), SwiGLU, then grouped GEMM2 (down), sharing
// one permuted input and one set of expert offsets.  Here:
//   * w13 mode: all micro-shards in ONE launch (the B operand is picked per
//     (micro, expert)); the A rows are gathered straight from x through
//     perm[p] / k, so the permuted input is never materialised; each tile
//     loads gate rows and the matching up rows of w1 so the SwiGLU
//     (SiLU(gate) * up, "HunyuanImage-3.0 on CANN NPU", section 2.2) is
//     applied in registers before the single rounding of h.
//   * down mode: the K loop runs over all micros' intermediate columns; the B
//     pointer switches micro at each Im boundary, so the per-micro partials
//     are summed in the fp32 accumulator and never exist as tensors.
//
// Work decomposition: a logical tile is (expert e, n-tile, m-tile of BM rows
// of e's segment), numbered expert-major, then n-tile, then m-tile, so
// neighbouring tiles share the same weight tile.  The expert counts live
// only on the device, so every workgroup decodes its tile from `offsets` with
// one wave scan; the grid is sized for the worst case and surplus workgroups
// exit.  Workgroups are dealt to the 8 XCDs round-robin by hardware; the
// remap below gives each XCD one contiguous range of logical tiles, so the
// workgroups that share a weight tile run on the same XCD and share its L2.
#include "moe_common.h"

namespace moe {
namespace {

enum Mode { kW13 = 0, kDown = 1 };

struct TileInfo {
  int e, m0, seg_end, nt, valid;
};

// Decode the logical tile of this workgroup.  Must be called by all threads;
// wave 0 computes, the result is broadcast through LDS.
template <int BM>
__device__ __forceinline__ TileInfo decode_tile(const int32_t* __restrict__ offsets, int E,
                                                int n_tiles) {
  __shared__ int s_info[5];
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int off = 0, cnt = 0;
    if (lane < E) {
      off = offsets[lane];
      cnt = offsets[lane + 1] - off;
    }
    const int mt = (cnt + BM - 1) / BM;
    const int tiles = mt * n_tiles;
    int incl = tiles;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int total = __shfl(incl, kWave - 1);
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int L = xcd * per + slot;
    const bool ok = slot < per && L < total;
    const uint64_t hit = __ballot(lane < E && incl > L);
    const int e = ok && hit ? (__ffsll((long long)hit) - 1) : 0;
    const int e_incl = __shfl(incl, e), e_tiles = __shfl(tiles, e), e_mt = __shfl(mt, e);
    const int e_off = __shfl(off, e), e_cnt = __shfl(cnt, e);
    if (lane == 0) {
      if (!ok || hit == 0) {
        s_info[4] = 0;
      } else {
        const int local = L - (e_incl - e_tiles);
        s_info[0] = e;
        s_info[1] = e_off + (local % e_mt) * BM;
        s_info[2] = e_off + e_cnt;
        s_info[3] = local / e_mt;
        s_info[4] = 1;
      }
    }
  }
  __syncthreads();
  TileInfo ti;
  ti.e = s_info[0];
  ti.m0 = s_info[1];
  ti.seg_end = s_info[2];
  ti.nt = s_info[3];
  ti.valid = s_info[4];
  return ti;
}

// ---------------------------------------------------------------------------
// bf16 MFMA path (v_mfma_f32_16x16x32_bf16).
//
// Tile: BM = 128 permuted rows x 256 B-rows (w13: 128 gate + 128 up rows ->
// 128 h columns; down: 256 output columns), BK = 64, four waves in a 2 x 2
// grid, each owning 64 rows x 128 B-rows = 4 x 8 MFMA blocks of 16 x 16.
// LDS holds two stages of A and B; global tiles are prefetched into registers
// during the MFMAs of the current stage.  LDS rows are padded to 72 bf16
// (144 B) so the 16-byte fragment reads of 16 consecutive rows hit distinct
// banks.

constexpr int BM = 128;
constexpr int BNB = 256;
constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int NTHR = 256;
constexpr int kStage = (BM + BNB) * LDK;  // bf16 elements per LDS stage

template <int MODE>
__global__ __launch_bounds__(NTHR, 1) void grouped_gemm_bf16(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int H, int E, int k, int Im, int mu, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * kStage];

  const TileInfo ti = decode_tile<BM>(offsets, E, n_tiles);
  if (!ti.valid) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lda = (MODE == kW13) ? H : mu * Im;
  const int K = lda;
  const int KT = K / BK;
  const int cc = tid & 7;       // 16-byte column chunk this thread copies
  const int rbase = tid >> 3;   // first tile row this thread copies

  // micro and column base of the n-tile
  int micro = 0, n0 = 0;
  if (MODE == kW13) {
    const int per_micro = Im / 128;
    micro = ti.nt / per_micro;
    n0 = (ti.nt % per_micro) * 128;
  } else {
    n0 = ti.nt * BNB;
  }

  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = min(ti.m0 + rbase + 32 * i, ti.seg_end - 1);
    if (MODE == kW13) {
      const int tok = perm[p] / k;
      a_src[i] = A + (size_t)tok * H + cc * 8;
    } else {
      a_src[i] = A + (size_t)p * lda + cc * 8;
    }
  }
  size_t b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int br = rbase + 32 * i;
    if (MODE == kW13) {
      const int wrow = br < 128 ? n0 + br : Im + n0 + (br - 128);
      b_off[i] = ((size_t)(micro * E + ti.e) * (2 * Im) + wrow) * H + cc * 8;
    } else {
      b_off[i] = ((size_t)ti.e * H + n0 + br) * Im + cc * 8;
    }
  }

  uint4 ra[4], rb[8];
  auto load_tile = [&](int kt) {
    const int kg = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + kg);
    if (MODE == kW13) {
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[i] = *reinterpret_cast<const uint4*>(B + b_off[i] + kg);
    } else {
      const int mm = kg / Im, kk = kg - mm * Im;
      const uint16_t* bm = B + (size_t)mm * E * H * Im + kk;
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[i] = *reinterpret_cast<const uint4*>(bm + b_off[i]);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* s = sm + buf * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(s + (rbase + 32 * i) * LDK + cc * 8) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(s + (BM + rbase + 32 * i) * LDK + cc * 8) = rb[i];
  };

  const int wm = wave & 1, wn = wave >> 1;
  const int frow = lane & 15, fk = (lane >> 4) * 8;
  int b_row[8];
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) {
    if (MODE == kW13)
      b_row[jb] = (jb < 4 ? wn * 64 + 16 * jb : 128 + wn * 64 + 16 * (jb - 4)) + frow;
    else
      b_row[jb] = wn * 128 + 16 * jb + frow;
  }

  f32x4 acc[4][8];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) acc[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) load_tile(kt + 1);
    const uint16_t* s = sm + (kt & 1) * kStage;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8 af[4], bfr[8];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        af[ib] = *reinterpret_cast<const bf16x8*>(s + (wm * 64 + 16 * ib + frow) * LDK + ks + fk);
#pragma unroll
      for (int jb = 0; jb < 8; ++jb)
        bfr[jb] = *reinterpret_cast<const bf16x8*>(s + (BM + b_row[jb]) * LDK + ks + fk);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
          acc[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ib], bfr[jb], acc[ib][jb], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile((kt + 1) & 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane>>4) + r, column lane & 15 of each block
  const int ldc = (MODE == kW13) ? mu * Im : H;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = ti.m0 + wm * 64 + 16 * ib + 4 * (lane >> 4) + r;
      if (p >= ti.seg_end) continue;
      uint16_t* crow = C + (size_t)p * ldc;
      if (MODE == kW13) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const float g = acc[ib][jb][r], u = acc[ib][jb + 4][r];
          crow[micro * Im + n0 + wn * 64 + 16 * jb + frow] = float_to_bf16_bits(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
          crow[n0 + wn * 128 + 16 * jb + frow] = float_to_bf16_bits(acc[ib][jb][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: plain LDS-tiled FMA GEMM (64 rows x 64 B-rows, BK = 16), each
// thread 4 rows x 4 B-rows.  In w13 mode a thread's four B-rows are two gate
// rows and the two matching up rows, so SwiGLU is applied in registers.

constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(
    const float* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const float* __restrict__ B, float* __restrict__ C,
    int H, int E, int k, int Im, int mu, int n_tiles) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];

  const TileInfo ti = decode_tile<FBM>(offsets, E, n_tiles);
  if (!ti.valid) return;

  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int lda = (MODE == kW13) ? H : mu * Im;
  const int K = lda;

  int micro = 0, n0 = 0;
  if (MODE == kW13) {
    const int per_micro = Im / 32;
    micro = ti.nt / per_micro;
    n0 = (ti.nt % per_micro) * 32;
  } else {
    n0 = ti.nt * FBN;
  }

  // loader: row lr = tid / 4, k-chunk lk = (tid % 4) * 4
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const float* a_src;
  {
    const int p = min(ti.m0 + lr, ti.seg_end - 1);
    a_src = (MODE == kW13) ? A + (size_t)(perm[p] / k) * H : A + (size_t)p * lda;
  }
  size_t b_base;
  if (MODE == kW13) {
    const int wrow = lr < 32 ? n0 + lr : Im + n0 + (lr - 32);
    b_base = ((size_t)(micro * E + ti.e) * (2 * Im) + wrow) * H;
  } else {
    b_base = ((size_t)ti.e * H + n0 + lr) * Im;
  }

  // B columns of this thread (indices into the 64 B-rows of the tile)
  int bc[4];
  if (MODE == kW13) {
    bc[0] = tx * 2; bc[1] = tx * 2 + 1; bc[2] = 32 + tx * 2; bc[3] = 32 + tx * 2 + 1;
  } else {
    bc[0] = tx * 4; bc[1] = tx * 4 + 1; bc[2] = tx * 4 + 2; bc[3] = tx * 4 + 3;
  }

  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    const float4 av = *reinterpret_cast<const float4*>(a_src + k0 + lk);
    float4 bv;
    if (MODE == kW13) {
      bv = *reinterpret_cast<const float4*>(B + b_base + k0 + lk);
    } else {
      const int mm = k0 / Im, kk = k0 - mm * Im;
      bv = *reinterpret_cast<const float4*>(B + (size_t)mm * E * H * Im + b_base + kk + lk);
    }
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][bc[j]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  const int ldc = (MODE == kW13) ? mu * Im : H;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = ti.m0 + ty * 4 + i;
    if (p >= ti.seg_end) continue;
    float* crow = C + (size_t)p * ldc;
    if (MODE == kW13) {
      crow[micro * Im + n0 + tx * 2] = silu_f32(acc[i][0]) * acc[i][2];
      crow[micro * Im + n0 + tx * 2 + 1] = silu_f32(acc[i][1]) * acc[i][3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) crow[n0 + bc[j]] = acc[i][j];
    }
  }
}

// Upper bound of sum_e ceil(count_e / bm) over any routing of R routes.
inline long long max_m_tiles(long long R, int E, int bm) {
  const long long a = (R + (long long)E * (bm - 1)) / bm;
  return a < 1 ? 1 : a;
}

inline unsigned grid_size(long long tiles) {
  const long long g = (tiles + kXcds - 1) / kXcds * kXcds;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_w13_swiglu(const Shape& s, const void* x, const int32_t* perm,
                             const int32_t* offsets, const void* w1, void* h, hipStream_t st) {
  if (s.bf16) {
    const int n_tiles = s.mu * (s.Im / 128);
    const unsigned g = grid_size(max_m_tiles(s.R(), s.E, BM) * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_bf16<kW13>, dim3(g), dim3(NTHR), 0, st, (const uint16_t*)x,
                       perm, offsets, (const uint16_t*)w1, (uint16_t*)h, s.H, s.E, s.k, s.Im,
                       s.mu, n_tiles);
  } else {
    const int n_tiles = s.mu * (s.Im / 32);
    const unsigned g = grid_size(max_m_tiles(s.R(), s.E, FBM) * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_f32<kW13>, dim3(g), dim3(256), 0, st, (const float*)x, perm,
                       offsets, (const float*)w1, (float*)h, s.H, s.E, s.k, s.Im, s.mu, n_tiles);
  }
  return hipGetLastError();
}

hipError_t launch_down(const Shape& s, const void* h, const int32_t* offsets, const void* w2,
                       void* y, hipStream_t st) {
  if (s.bf16) {
    const int n_tiles = s.H / BNB;
    const unsigned g = grid_size(max_m_tiles(s.R(), s.E, BM) * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_bf16<kDown>, dim3(g), dim3(NTHR), 0, st, (const uint16_t*)h,
                       nullptr, offsets, (const uint16_t*)w2, (uint16_t*)y, s.H, s.E, s.k, s.Im,
                       s.mu, n_tiles);
  } else {
    const int n_tiles = s.H / FBN;
    const unsigned g = grid_size(max_m_tiles(s.R(), s.E, FBM) * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_f32<kDown>, dim3(g), dim3(256), 0, st, (const float*)h,
                       nullptr, offsets, (const float*)w2, (float*)y, s.H, s.E, s.k, s.Im, s.mu,
                       n_tiles);
  }
  return hipGetLastError();
}

}  // namespace moe
