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
//     are summed in the fp32 accumulator and never exist as tensors; y
//     leaves as that fp32 accumulator (no rounding before the finalize).
//
// Work decomposition: a logical tile is (expert e, n-tile, m-tile of BM rows
// of e's segment), numbered expert-major, then n-tile, then m-tile, so
// neighbouring tiles share the same weight tile.  The expert counts live
// only on the device, so every workgroup decodes its tile from `offsets` with
// one wave scan; the grid is sized for the worst case and surplus workgroups
// exit.  Workgroups are dealt to the 8 XCDs round-robin by hardware; the
// remap below gives each XCD one contiguous range of logical tiles, so the
// workgroups that share a weight tile run on the same XCD and share its L2.
#include "gemm_fast.h"
#include "moe_common.h"

namespace moe {
namespace {

using fast::kDown;
using fast::kW13;

// ---------------------------------------------------------------------------
// fp32 path: plain LDS-tiled FMA GEMM (64 rows x 64 B-rows, BK = 16), each
// thread 4 rows x 4 B-rows.  In w13 mode a thread's four B-rows are two gate
// rows and the two matching up rows, so SwiGLU is applied in registers.

constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(
    const float* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const float* __restrict__ B, float* __restrict__ C,
    int H, int E, int k, int Im, int mu, int n_tiles, int dense_rows) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];

  const fast::Tile ti = fast::decode<FBM>(offsets, E, n_tiles, dense_rows);
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
    if constexpr (MODE == kW13) {
      const int xr = offsets == nullptr ? p : perm[p] / k;  // dense segment: x row p
      a_src = A + (size_t)xr * H;
    } else {
      a_src = A + (size_t)p * lda;  // down: row p of h (no perm is passed)
    }
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

// bf16 tile configurations (measured on MI355X for the denoise layer, the
// variants interleaved in one process on random data):
// w13: 320 rows x (128 gate + 128 up) B-rows, BK 64, 8 waves of 80 x 128
// (4 x 2 waves: 13 fragment reads per 40 MFMAs instead of 14 for 160 x 64,
// and a partial tile's padded rows skipped in 80-row blocks; 3% faster, h
// bit-identical); down: 320 rows x 256 output columns, 8 waves of 80 x 128
// (5% faster than 256 rows in 2 x 4 waves of 128 x 64; 320 rows in 2 x 4
// were not).  BK 64 keeps
// every row copy a full 128-byte line (64-byte pieces halve the copy rate).
// Two waves per SIMD are needed for the 16x16x32 MFMA to issue at full rate.
//  * 320-row tiles cover an expert of up to 640 routes in two m-tiles (256-row
//    tiles need three once an expert passes 512, and each extra m-tile streams
//    the expert's weight tile again): 2.3% faster for w13 at the near-uniform
//    loads of the denoise layer (6% with the 4 x 2 waves).
//  * Two weight slots for both.  A third slot raised w13's fabric reads by
//    16% for no gain; for down it helped while the epilogue stored 32-byte
//    pieces, and is 2% slower since the epilogue goes through LDS (down's
//    output tile leaves in one pass per 80-row block of waves).
using W13Cfg = fast::Cfg<fast::kW13, 320, 256, 64, 2, 4, 2, 2>;
using DownCfg = fast::Cfg<fast::kDown, 320, 256, 64, 2, 4, 2, 2>;
// Narrower shapes of the envelope (none of the benchmark's layers): w13 tiles
// of 32 gate + 32 up columns when Im (or the shared width) is not a multiple
// of 128, and down k-steps of 32 when it is not a multiple of 64, so that no
// k-step crosses a micro-shard boundary (256-row tiles: a 1 KB copy covers 16
// rows of 64 bytes, and 320 rows do not split evenly over the 8 waves).
using W13NarrowCfg = fast::Cfg<fast::kW13, 320, 64, 64, 2, 4, 2, 2>;
using DownK32Cfg = fast::Cfg<fast::kDown, 256, 256, 32, 2, 4, 2, 2>;

inline bool wide_w13(int w) { return w % W13Cfg::HCOLS == 0; }
inline bool deep_down(int w) { return w % DownCfg::BK == 0; }


inline unsigned grid_size(long long tiles) {
  const long long g = (tiles + kXcds - 1) / kXcds * kXcds;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_w13_swiglu(const Shape& s, const void* x, const int32_t* perm,
                             const int32_t* offsets, const void* w1, void* h, hipStream_t st) {
  if (s.bf16) {
    if (wide_w13(s.Im)) return fast::launch<W13Cfg>(x, perm, offsets, w1, h, s.T, s.H, s.E, s.k, s.Im, s.mu, st);
    return fast::launch<W13NarrowCfg>(x, perm, offsets, w1, h, s.T, s.H, s.E, s.k, s.Im, s.mu, st);
  } else {
    const int n_tiles = s.mu * (s.Im / 32);
    const unsigned g = grid_size(fast::max_m_tiles(s.R(), s.E, FBM) * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_f32<kW13>, dim3(g), dim3(256), 0, st, (const float*)x, perm,
                       offsets, (const float*)w1, (float*)h, s.H, s.E, s.k, s.Im, s.mu, n_tiles, s.T);
  }
  return hipGetLastError();
}

hipError_t launch_w13_swiglu_with_dense(const Shape& s, const void* x, const int32_t* perm,
                                        const int32_t* offsets, const void* w1, void* h,
                                        const void* w1d, void* hd, int wd, hipStream_t st) {
  const fast::Extra ex{(const uint16_t*)x, (const uint16_t*)w1d, hd, s.T, wd};
  if (wide_w13(s.Im) && wide_w13(wd))
    return fast::launch<W13Cfg>(x, perm, offsets, w1, h, s.T, s.H, s.E, s.k, s.Im, s.mu, st, ex);
  return fast::launch<W13NarrowCfg>(x, perm, offsets, w1, h, s.T, s.H, s.E, s.k, s.Im, s.mu, st, ex);
}

hipError_t launch_down_with_dense(const Shape& s, const void* h, const int32_t* offsets,
                                  const void* w2, void* y, const void* hd, const void* w2d,
                                  void* yd, int wd, hipStream_t st) {
  const fast::Extra ex{(const uint16_t*)hd, (const uint16_t*)w2d, yd, s.T, wd};
  if (deep_down(s.Im) && deep_down(wd))
    return fast::launch<DownCfg>(h, nullptr, offsets, w2, y, s.T, s.H, s.E, s.k, s.Im, s.mu, st, ex);
  return fast::launch<DownK32Cfg>(h, nullptr, offsets, w2, y, s.T, s.H, s.E, s.k, s.Im, s.mu, st, ex);
}

hipError_t launch_down(const Shape& s, const void* h, const int32_t* offsets, const void* w2,
                       void* y, hipStream_t st) {
  if (s.bf16) {
    if (deep_down(s.Im)) return fast::launch<DownCfg>(h, nullptr, offsets, w2, y, s.T, s.H, s.E, s.k, s.Im, s.mu, st);
    return fast::launch<DownK32Cfg>(h, nullptr, offsets, w2, y, s.T, s.H, s.E, s.k, s.Im, s.mu, st);
  } else {
    const int n_tiles = s.H / FBN;
    const unsigned g = grid_size(fast::max_m_tiles(s.R(), s.E, FBM) * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_f32<kDown>, dim3(g), dim3(256), 0, st, (const float*)h,
                       nullptr, offsets, (const float*)w2, (float*)y, s.H, s.E, s.k, s.Im, s.mu,
                       n_tiles, s.T);
  }
  return hipGetLastError();
}

}  // namespace moe
