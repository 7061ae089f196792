// Pipelined bf16 MFMA grouped GEMM for the expert FFN (gfx950).
//
// Same contract as the grouped GEMMs of gemm.hip (w13 mode: gathered rows of
// x times gate|up rows of w1 with the SwiGLU epilogue; down mode: h rows
// times w2 rows with micro-shards summed in the accumulator), restructured
// for throughput:
//   * global -> LDS copies use the CDNA4 direct-to-LDS load
//     (global_load_lds_dwordx4): no staging registers, no LDS write
//     instructions; STAGES tiles are in flight while the MFMAs consume one.
//   * LDS rows are BK bf16 long with their 16-byte chunks XOR-swizzled per
//     row, so the 16 rows read by one MFMA fragment load hit 16 distinct
//     16-byte bank groups.
//   * WM x WN waves, each owning a (BM/WM) x (BN/WN) block of 16x16 MFMA
//     tiles (v_mfma_f32_16x16x32_bf16), accumulators in AGPRs.
#pragma once

#include "moe_common.h"

namespace moe {
namespace fast {

enum Mode { kW13 = 0, kDown = 1 };

typedef __attribute__((address_space(3))) void lds_void;

template <int MODE_, int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_>
struct Cfg {
  static constexpr int MODE = MODE_, BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN;
  static constexpr int NTHR = NW * 64;
  static constexpr int TM = BM / WM;    // rows per wave
  static constexpr int TN = BN / WN;    // B-rows per wave
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int CPR = BK / 8;    // 16-byte chunks per LDS row
  static constexpr int RPI = 64 / CPR;  // rows per 1 KB direct-to-LDS load
  static constexpr int A_PER_WAVE = BM / RPI / NW;
  static constexpr int B_PER_WAVE = BN / RPI / NW;
  static constexpr int NI = A_PER_WAVE + B_PER_WAVE;  // loads per wave per stage
  static constexpr int STAGE = (BM + BN) * BK;        // bf16 elements per stage
  static constexpr int LDS_BYTES = STAGES * STAGE * 2;
  static constexpr int HCOLS = (MODE == kW13) ? BN / 2 : BN;  // output columns per tile
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "load split");
  static_assert(TM % 16 == 0 && TN % 32 == 0, "wave tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// swizzle of the 16-byte chunk index within a row
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  return (row / (16 / CPR)) % CPR;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // s_waitcnt with only vmcnt restricted (expcnt = 7, lgkmcnt = 15: no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One direct-to-LDS load: every lane copies 16 bytes from sbase + voff (bytes)
// to LDS address lds + 16 * lane.  Issued as inline asm so the compiler's
// wait-count tracking does not serialise the pipeline: callers wait on vmcnt
// and barrier themselves before reading the destination.
__device__ __forceinline__ void dma16(uint32_t lds, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory");
}

struct Tile {
  int e, m0, seg_end, nt, valid;
};

// Logical tile of this workgroup (expert-major, then n-tile, then m-tile),
// decoded from the device-side offsets; XCD-aware: XCD x (= blockIdx % 8)
// takes the contiguous logical range [x*per, (x+1)*per).
template <int BM>
__device__ __forceinline__ Tile decode(const int32_t* __restrict__ offsets, int E, int n_tiles) {
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
  Tile t;
  t.e = s_info[0];
  t.m0 = s_info[1];
  t.seg_end = s_info[2];
  t.nt = s_info[3];
  t.valid = s_info[4];
  return t;
}

template <class C>
__global__ __launch_bounds__(C::NTHR, 1) void grouped_gemm(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B, uint16_t* __restrict__ Cout,
    int H, int E, int k, int Im, int mu, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::STAGES * C::STAGE];

  const Tile ti = decode<C::BM>(offsets, E, n_tiles);
  if (!ti.valid) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lda = (C::MODE == kW13) ? H : mu * Im;
  const int KT = lda / C::BK;

  int micro = 0, n0 = 0;
  if (C::MODE == kW13) {
    const int per_micro = Im / C::HCOLS;
    micro = ti.nt / per_micro;
    n0 = (ti.nt % per_micro) * C::HCOLS;
  } else {
    n0 = ti.nt * C::BN;
  }

  // ---- per-lane byte offsets of the direct-to-LDS loads
  // load i of this wave covers tile rows [g*RPI, (g+1)*RPI), g = wave + NW*i;
  // lane -> row g*RPI + lane/CPR, LDS chunk lane%CPR, logical chunk ^ swz.
  const int lrow = lane / C::CPR;
  const int lpos = lane % C::CPR;
  uint32_t a_off[C::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; ++i) {
    const int row = (wave + C::NW * i) * C::RPI + lrow;
    const int c = lpos ^ swz<C::CPR>(row);
    const int p = min(ti.m0 + row, ti.seg_end - 1);
    const uint32_t r = (C::MODE == kW13) ? (uint32_t)(perm[p] / k) * (uint32_t)H : (uint32_t)p * (uint32_t)lda;
    a_off[i] = (r + c * 8) * 2u;
  }
  const uint16_t* b_base;
  uint32_t b_ld;
  if (C::MODE == kW13) {
    b_base = B + (size_t)(micro * E + ti.e) * (2 * Im) * H;
    b_ld = H;
  } else {
    b_base = B + ((size_t)ti.e * H + n0) * Im;
    b_ld = Im;
  }
  uint32_t b_off[C::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::B_PER_WAVE; ++i) {
    const int row = (wave + C::NW * i) * C::RPI + lrow;
    const int c = lpos ^ swz<C::CPR>(row);
    int wrow = row;
    if (C::MODE == kW13) wrow = row < C::BN / 2 ? n0 + row : Im + n0 + (row - C::BN / 2);
    b_off[i] = ((uint32_t)wrow * b_ld + c * 8) * 2u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  auto issue = [&](int kt, int stage) {
    const int kg = kt * C::BK;
    const uint32_t sb = lds0 + (uint32_t)(stage * C::STAGE) * 2u;
    const uint16_t* abase = A + kg;
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((wave + C::NW * i) * C::RPI * C::BK) * 2u, abase, a_off[i]);
    const uint16_t* bbase = b_base + kg;
    if (C::MODE == kDown) {
      const int mm = kg / Im;
      bbase = b_base + (size_t)mm * E * H * Im + (kg - mm * Im);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((C::BM + (wave + C::NW * i) * C::RPI) * C::BK) * 2u, bbase, b_off[i]);
  };

  // ---- MFMA fragment addressing (row = 16-aligned base + lane%16)
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int fr = lane & 15;
  const int sw = swz<C::CPR>(fr);
  int fa[C::FM], fb[C::FN];
#pragma unroll
  for (int f = 0; f < C::FM; ++f) fa[f] = (wm * C::TM + 16 * f + fr) * C::BK;
#pragma unroll
  for (int f = 0; f < C::FN; ++f) {
    int r;
    if (C::MODE == kW13)
      r = (f < C::FN / 2) ? wn * (C::TN / 2) + 16 * f : C::BN / 2 + wn * (C::TN / 2) + 16 * (f - C::FN / 2);
    else
      r = wn * C::TN + 16 * f;
    fb[f] = (C::BM + r + fr) * C::BK;
  }

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) issue(s, s);

  for (int kt = 0; kt < KT; ++kt) {
    if (kt + C::STAGES - 2 < KT)
      wait_vmcnt<(C::STAGES - 2) * C::NI>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (kt + C::STAGES - 1 < KT) issue(kt + C::STAGES - 1, (kt + C::STAGES - 1) % C::STAGES);
    const uint16_t* s = smem + (kt % C::STAGES) * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      const int ch = ((ks * 4 + (lane >> 4)) ^ sw) * 8;
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int f = 0; f < C::FM; ++f) af[f] = *reinterpret_cast<const bf16x8*>(s + fa[f] + ch);
#pragma unroll
      for (int f = 0; f < C::FN; ++f) bfr[f] = *reinterpret_cast<const bf16x8*>(s + fb[f] + ch);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane holds rows 4*(lane>>4)+r, column lane&15 of each block
  const int ldc = (C::MODE == kW13) ? mu * Im : H;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = ti.m0 + wm * C::TM + 16 * i + 4 * (lane >> 4) + r;
      if (p >= ti.seg_end) continue;
      uint16_t* crow = Cout + (size_t)p * ldc;
      if (C::MODE == kW13) {
#pragma unroll
        for (int j = 0; j < C::FN / 2; ++j) {
          const float g = acc[i][j][r], u = acc[i][j + C::FN / 2][r];
          crow[micro * Im + n0 + wn * (C::TN / 2) + 16 * j + fr] = float_to_bf16_bits(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          crow[n0 + wn * C::TN + 16 * j + fr] = float_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

// Wave-local tile decode: every wave computes the same result from the
// offsets with its own 64-lane scan, so no LDS slot or barrier is needed.
template <int BM>
__device__ __forceinline__ Tile decode_wave(const int32_t* __restrict__ offsets, int E, int n_tiles) {
  const int lane = threadIdx.x & 63;
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
  Tile t;
  t.valid = (ok && hit) ? 1 : 0;
  const int local = L - (e_incl - e_tiles);
  t.e = e;
  t.m0 = e_off + (t.valid ? (local % e_mt) * BM : 0);
  t.seg_end = e_off + e_cnt;
  t.nt = t.valid ? local / e_mt : 0;
  t.valid = __builtin_amdgcn_readfirstlane(t.valid);
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
  t.seg_end = __builtin_amdgcn_readfirstlane(t.seg_end);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  return t;
}

// Split-role variant: the weight operand B streams from HBM on first touch
// and needs more bytes in flight than the gathered activations A (served
// from L2 / infinity cache), so B gets SB ring slots and A only SA.  vmcnt
// retires in issue order, so one wave cannot wait for its A copy while its
// later B copies stay in flight; instead the first half of the waves copies
// only A and the second half only B, each waiting on its own counter.
template <int MODE_, int BM_, int BN_, int BK_, int SA_, int SB_, int WM_, int WN_>
struct SplitCfg {
  static constexpr int MODE = MODE_, BM = BM_, BN = BN_, BK = BK_, SA = SA_, SB = SB_;
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN;
  static constexpr int NTHR = NW * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int CPR = BK / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int HALF = NW / 2;
  static constexpr int A_PER_WAVE = BM / RPI / HALF;
  static constexpr int B_PER_WAVE = BN / RPI / HALF;
  static constexpr int A_STAGE = BM * BK, B_STAGE = BN * BK;  // bf16 elements
  static constexpr int LDS_BYTES = (SA * A_STAGE + SB * B_STAGE) * 2;
  static constexpr int HCOLS = (MODE == kW13) ? BN / 2 : BN;
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(SA >= 2 && SB >= 2, "stages");
  static_assert(BM % (RPI * HALF) == 0 && BN % (RPI * HALF) == 0, "load split");
  static_assert(TM % 16 == 0 && TN % 32 == 0, "wave tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <class C>
__global__ __launch_bounds__(C::NTHR, 1) void grouped_gemm_split(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B, uint16_t* __restrict__ Cout,
    int H, int E, int k, int Im, int mu, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::SA * C::A_STAGE + C::SB * C::B_STAGE];

  const Tile ti = decode_wave<C::BM>(offsets, E, n_tiles);
  if (!ti.valid) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool a_role = wave < C::HALF;
  const int rw = a_role ? wave : wave - C::HALF;  // index among the waves of this role
  const int lda = (C::MODE == kW13) ? H : mu * Im;
  const int KT = lda / C::BK;

  int micro = 0, n0 = 0;
  if (C::MODE == kW13) {
    const int per_micro = Im / C::HCOLS;
    micro = ti.nt / per_micro;
    n0 = (ti.nt % per_micro) * C::HCOLS;
  } else {
    n0 = ti.nt * C::BN;
  }

  const int lrow = lane / C::CPR;
  const int lpos = lane % C::CPR;
  constexpr int NL = C::A_PER_WAVE > C::B_PER_WAVE ? C::A_PER_WAVE : C::B_PER_WAVE;
  uint32_t off[NL];
  const uint16_t* b_base;
  if (C::MODE == kW13)
    b_base = B + (size_t)(micro * E + ti.e) * (2 * Im) * H;
  else
    b_base = B + ((size_t)ti.e * H + n0) * Im;
  if (a_role) {
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i) {
      const int row = (rw + C::HALF * i) * C::RPI + lrow;
      const int c = lpos ^ swz<C::CPR>(row);
      const int p = min(ti.m0 + row, ti.seg_end - 1);
      const uint32_t r = (C::MODE == kW13) ? (uint32_t)(perm[p] / k) * (uint32_t)H : (uint32_t)p * (uint32_t)lda;
      off[i] = (r + c * 8) * 2u;
    }
  } else {
    const uint32_t b_ld = (C::MODE == kW13) ? H : Im;
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i) {
      const int row = (rw + C::HALF * i) * C::RPI + lrow;
      const int c = lpos ^ swz<C::CPR>(row);
      int wrow = row;
      if (C::MODE == kW13) wrow = row < C::BN / 2 ? n0 + row : Im + n0 + (row - C::BN / 2);
      off[i] = ((uint32_t)wrow * b_ld + c * 8) * 2u;
    }
  }
  const uint32_t ldsA = (uint32_t)(uintptr_t)smem;
  const uint32_t ldsB = ldsA + (uint32_t)(C::SA * C::A_STAGE) * 2u;

  auto issue_a = [&](int kt) {
    const uint32_t sb = ldsA + (uint32_t)((kt % C::SA) * C::A_STAGE) * 2u;
    const uint16_t* abase = A + kt * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((rw + C::HALF * i) * C::RPI * C::BK) * 2u, abase, off[i]);
  };
  auto issue_b = [&](int kt) {
    const int kg = kt * C::BK;
    const uint32_t sb = ldsB + (uint32_t)((kt % C::SB) * C::B_STAGE) * 2u;
    const uint16_t* bbase = b_base + kg;
    if (C::MODE == kDown) {
      const int mm = kg / Im;
      bbase = b_base + (size_t)mm * E * H * Im + (kg - mm * Im);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((rw + C::HALF * i) * C::RPI * C::BK) * 2u, bbase, off[i]);
  };

  const int wm = wave % C::WM, wn = wave / C::WM;
  const int fr = lane & 15;
  const int sw = swz<C::CPR>(fr);
  int fa[C::FM], fb[C::FN];
#pragma unroll
  for (int f = 0; f < C::FM; ++f) fa[f] = (wm * C::TM + 16 * f + fr) * C::BK;
#pragma unroll
  for (int f = 0; f < C::FN; ++f) {
    int r;
    if (C::MODE == kW13)
      r = (f < C::FN / 2) ? wn * (C::TN / 2) + 16 * f : C::BN / 2 + wn * (C::TN / 2) + 16 * (f - C::FN / 2);
    else
      r = wn * C::TN + 16 * f;
    fb[f] = (r + fr) * C::BK;
  }

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: A stages 0 .. SA-2, B stages 0 .. SB-2
  if (a_role) {
#pragma unroll
    for (int s = 0; s < C::SA - 1; ++s)
      if (s < KT) issue_a(s);
  } else {
#pragma unroll
    for (int s = 0; s < C::SB - 1; ++s)
      if (s < KT) issue_b(s);
  }

  for (int kt = 0; kt < KT; ++kt) {
    // stage kt of this wave's operand must have landed; later stages may fly
    if (a_role) {
      if (kt + C::SA - 2 < KT) wait_vmcnt<(C::SA - 2) * C::A_PER_WAVE>(); else wait_vmcnt<0>();
    } else {
      if (kt + C::SB - 2 < KT) wait_vmcnt<(C::SB - 2) * C::B_PER_WAVE>(); else wait_vmcnt<0>();
    }
    __syncthreads();
    // refill the slot read in iteration kt-1 (every wave passed that barrier)
    if (a_role) {
      if (kt + C::SA - 1 < KT) issue_a(kt + C::SA - 1);
    } else {
      if (kt + C::SB - 1 < KT) issue_b(kt + C::SB - 1);
    }
    const uint16_t* sa = smem + (kt % C::SA) * C::A_STAGE;
    const uint16_t* sbp = smem + C::SA * C::A_STAGE + (kt % C::SB) * C::B_STAGE;
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      const int ch = ((ks * 4 + (lane >> 4)) ^ sw) * 8;
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int f = 0; f < C::FM; ++f) af[f] = *reinterpret_cast<const bf16x8*>(sa + fa[f] + ch);
#pragma unroll
      for (int f = 0; f < C::FN; ++f) bfr[f] = *reinterpret_cast<const bf16x8*>(sbp + fb[f] + ch);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  const int ldc = (C::MODE == kW13) ? mu * Im : H;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = ti.m0 + wm * C::TM + 16 * i + 4 * (lane >> 4) + r;
      if (p >= ti.seg_end) continue;
      uint16_t* crow = Cout + (size_t)p * ldc;
      if (C::MODE == kW13) {
#pragma unroll
        for (int j = 0; j < C::FN / 2; ++j) {
          const float g = acc[i][j][r], u = acc[i][j + C::FN / 2][r];
          crow[micro * Im + n0 + wn * (C::TN / 2) + 16 * j + fr] = float_to_bf16_bits(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          crow[n0 + wn * C::TN + 16 * j + fr] = float_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

template <class C>
hipError_t launch_split(const void* a, const int32_t* perm, const int32_t* offsets, const void* b,
                        void* c, int T, int H, int E, int k, int Im, int mu, hipStream_t st);

// Variant on v_mfma_f32_32x32x16_bf16.  One wave per SIMD keeps the matrix
// pipe busy with these (measured: 83% of peak from a single wave, against
// 34% with 16x16x32), so a workgroup can use four waves with 128 x 128 wave
// tiles, which read a third fewer LDS bytes per MFMA than 128 x 64 tiles.
// Fragments: A 32 rows x 16 k (lane: row lane%32, k-chunk lane/32), B the
// same on B-rows; D: register i of lane holds row 8*(i/4) + 4*(lane/32) + i%4,
// column lane%32.
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class C>
__global__ __launch_bounds__(C::NTHR, 1) void grouped_gemm32(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B, uint16_t* __restrict__ Cout,
    int H, int E, int k, int Im, int mu, int n_tiles) {
  static_assert(C::TM % 32 == 0 && C::TN % 64 == 0, "32x32 wave tile");
  constexpr int FM = C::TM / 32, FN = C::TN / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::STAGES * C::STAGE];

  const Tile ti = decode<C::BM>(offsets, E, n_tiles);
  if (!ti.valid) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lda = (C::MODE == kW13) ? H : mu * Im;
  const int KT = lda / C::BK;

  int micro = 0, n0 = 0;
  if (C::MODE == kW13) {
    const int per_micro = Im / C::HCOLS;
    micro = ti.nt / per_micro;
    n0 = (ti.nt % per_micro) * C::HCOLS;
  } else {
    n0 = ti.nt * C::BN;
  }

  const int lrow = lane / C::CPR;
  const int lpos = lane % C::CPR;
  uint32_t a_off[C::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; ++i) {
    const int row = (wave + C::NW * i) * C::RPI + lrow;
    const int c = lpos ^ swz<C::CPR>(row);
    const int p = min(ti.m0 + row, ti.seg_end - 1);
    const uint32_t r = (C::MODE == kW13) ? (uint32_t)(perm[p] / k) * (uint32_t)H : (uint32_t)p * (uint32_t)lda;
    a_off[i] = (r + c * 8) * 2u;
  }
  const uint16_t* b_base;
  uint32_t b_ld;
  if (C::MODE == kW13) {
    b_base = B + (size_t)(micro * E + ti.e) * (2 * Im) * H;
    b_ld = H;
  } else {
    b_base = B + ((size_t)ti.e * H + n0) * Im;
    b_ld = Im;
  }
  uint32_t b_off[C::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::B_PER_WAVE; ++i) {
    const int row = (wave + C::NW * i) * C::RPI + lrow;
    const int c = lpos ^ swz<C::CPR>(row);
    int wrow = row;
    if (C::MODE == kW13) wrow = row < C::BN / 2 ? n0 + row : Im + n0 + (row - C::BN / 2);
    b_off[i] = ((uint32_t)wrow * b_ld + c * 8) * 2u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  auto issue = [&](int kt, int stage) {
    const int kg = kt * C::BK;
    const uint32_t sb = lds0 + (uint32_t)(stage * C::STAGE) * 2u;
    const uint16_t* abase = A + kg;
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((wave + C::NW * i) * C::RPI * C::BK) * 2u, abase, a_off[i]);
    const uint16_t* bbase = b_base + kg;
    if (C::MODE == kDown) {
      const int mm = kg / Im;
      bbase = b_base + (size_t)mm * E * H * Im + (kg - mm * Im);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((C::BM + (wave + C::NW * i) * C::RPI) * C::BK) * 2u, bbase, b_off[i]);
  };

  const int wm = wave % C::WM, wn = wave / C::WM;
  const int fr = lane & 31;
  const int sw = swz<C::CPR>(fr);
  int fa[FM], fb[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) fa[f] = (wm * C::TM + 32 * f + fr) * C::BK;
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    int r;
    if (C::MODE == kW13)
      r = (f < FN / 2) ? wn * (C::TN / 2) + 32 * f : C::BN / 2 + wn * (C::TN / 2) + 32 * (f - FN / 2);
    else
      r = wn * C::TN + 32 * f;
    fb[f] = (C::BM + r + fr) * C::BK;
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) issue(s, s);

  // one wave per SIMD: the fragments of k16-step ks+1 are read from LDS
  // while the MFMAs of step ks run, so LDS latency hides under the matrix pipe
  constexpr int KS = C::BK / 16;
  bf16x8 af[2][FM], bfr[2][FN];
  auto load_frags = [&](const uint16_t* st, int ks, int buf) {
    const int ch = ((ks * 2 + (lane >> 5)) ^ sw) * 8;
#pragma unroll
    for (int f = 0; f < FM; ++f) af[buf][f] = *reinterpret_cast<const bf16x8*>(st + fa[f] + ch);
#pragma unroll
    for (int f = 0; f < FN; ++f) bfr[buf][f] = *reinterpret_cast<const bf16x8*>(st + fb[f] + ch);
  };
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + C::STAGES - 2 < KT)
      wait_vmcnt<(C::STAGES - 2) * C::NI>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (kt + C::STAGES - 1 < KT) issue(kt + C::STAGES - 1, (kt + C::STAGES - 1) % C::STAGES);
    const uint16_t* st = smem + (kt % C::STAGES) * C::STAGE;
    load_frags(st, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load_frags(st, ks + 1, (ks + 1) & 1);
      // keep the next step's reads ahead of this step's MFMAs (the scheduler
      // would otherwise sink them to their use and expose LDS latency)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  const int ldc = (C::MODE == kW13) ? mu * Im : H;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int p = ti.m0 + wm * C::TM + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      if (p >= ti.seg_end) continue;
      uint16_t* crow = Cout + (size_t)p * ldc;
      if (C::MODE == kW13) {
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const float g = acc[i][j][q], u = acc[i][j + FN / 2][q];
          crow[micro * Im + n0 + wn * (C::TN / 2) + 32 * j + fr] = float_to_bf16_bits(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          crow[n0 + wn * C::TN + 32 * j + fr] = float_to_bf16_bits(acc[i][j][q]);
      }
    }
  }
}

// Variant with fragments double-buffered across k-tiles: while the MFMAs
// of k-tile kt run from registers, the fragments of k-tile kt+1 are read
// from LDS, so the matrix pipe does not drain at the per-tile barrier.
// Needs STAGES >= 4: at the end of iteration kt the stage kt+2 must have
// landed (its fragments are read during iteration kt+1), and the DMA issued
// at iteration kt targets the buffer of stage kt-1, whose fragments were
// read during iteration kt-2.
template <class C>
__global__ __launch_bounds__(C::NTHR, 1) void grouped_gemm_db(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B, uint16_t* __restrict__ Cout,
    int H, int E, int k, int Im, int mu, int n_tiles) {
  static_assert(C::STAGES >= 4, "double-buffered fragments need 4 stages");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::STAGES * C::STAGE];

  const Tile ti = decode<C::BM>(offsets, E, n_tiles);
  if (!ti.valid) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lda = (C::MODE == kW13) ? H : mu * Im;
  const int KT = lda / C::BK;

  int micro = 0, n0 = 0;
  if (C::MODE == kW13) {
    const int per_micro = Im / C::HCOLS;
    micro = ti.nt / per_micro;
    n0 = (ti.nt % per_micro) * C::HCOLS;
  } else {
    n0 = ti.nt * C::BN;
  }

  const int lrow = lane / C::CPR;
  const int lpos = lane % C::CPR;
  uint32_t a_off[C::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; ++i) {
    const int row = (wave + C::NW * i) * C::RPI + lrow;
    const int c = lpos ^ swz<C::CPR>(row);
    const int p = min(ti.m0 + row, ti.seg_end - 1);
    const uint32_t r = (C::MODE == kW13) ? (uint32_t)(perm[p] / k) * (uint32_t)H : (uint32_t)p * (uint32_t)lda;
    a_off[i] = (r + c * 8) * 2u;
  }
  const uint16_t* b_base;
  uint32_t b_ld;
  if (C::MODE == kW13) {
    b_base = B + (size_t)(micro * E + ti.e) * (2 * Im) * H;
    b_ld = H;
  } else {
    b_base = B + ((size_t)ti.e * H + n0) * Im;
    b_ld = Im;
  }
  uint32_t b_off[C::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::B_PER_WAVE; ++i) {
    const int row = (wave + C::NW * i) * C::RPI + lrow;
    const int c = lpos ^ swz<C::CPR>(row);
    int wrow = row;
    if (C::MODE == kW13) wrow = row < C::BN / 2 ? n0 + row : Im + n0 + (row - C::BN / 2);
    b_off[i] = ((uint32_t)wrow * b_ld + c * 8) * 2u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  auto issue = [&](int kt, int stage) {
    const int kg = kt * C::BK;
    const uint32_t sb = lds0 + (uint32_t)(stage * C::STAGE) * 2u;
    const uint16_t* abase = A + kg;
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((wave + C::NW * i) * C::RPI * C::BK) * 2u, abase, a_off[i]);
    const uint16_t* bbase = b_base + kg;
    if (C::MODE == kDown) {
      const int mm = kg / Im;
      bbase = b_base + (size_t)mm * E * H * Im + (kg - mm * Im);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((C::BM + (wave + C::NW * i) * C::RPI) * C::BK) * 2u, bbase, b_off[i]);
  };

  const int wm = wave % C::WM, wn = wave / C::WM;
  const int fr = lane & 15;
  const int sw = swz<C::CPR>(fr);
  int fa[C::FM], fb[C::FN];
#pragma unroll
  for (int f = 0; f < C::FM; ++f) fa[f] = (wm * C::TM + 16 * f + fr) * C::BK;
#pragma unroll
  for (int f = 0; f < C::FN; ++f) {
    int r;
    if (C::MODE == kW13)
      r = (f < C::FN / 2) ? wn * (C::TN / 2) + 16 * f : C::BN / 2 + wn * (C::TN / 2) + 16 * (f - C::FN / 2);
    else
      r = wn * C::TN + 16 * f;
    fb[f] = (C::BM + r + fr) * C::BK;
  }
  constexpr int KS = C::BK / 32;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa0[KS][C::FM], fb0[KS][C::FN], fa1[KS][C::FM], fb1[KS][C::FN];
  auto load_frags = [&](int kt, bf16x8 (&xa)[KS][C::FM], bf16x8 (&xb)[KS][C::FN]) {
    const uint16_t* s = smem + (kt % C::STAGES) * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = ((ks * 4 + (lane >> 4)) ^ sw) * 8;
#pragma unroll
      for (int f = 0; f < C::FM; ++f) xa[ks][f] = *reinterpret_cast<const bf16x8*>(s + fa[f] + ch);
#pragma unroll
      for (int f = 0; f < C::FN; ++f) xb[ks][f] = *reinterpret_cast<const bf16x8*>(s + fb[f] + ch);
    }
  };
  auto mfmas = [&](bf16x8 (&xa)[KS][C::FM], bf16x8 (&xb)[KS][C::FN]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[ks][i], xb[ks][j], acc[i][j], 0, 0, 0);
  };
  auto sync_end = [&](int kt) {
    // stage kt+2 must have landed for the fragment reads of iteration kt+1
    if (kt + C::STAGES - 1 < KT)
      wait_vmcnt<(C::STAGES - 3) * C::NI>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  };

#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) issue(s, s);
  if (C::STAGES - 1 <= KT)
    wait_vmcnt<(C::STAGES - 3) * C::NI>();
  else
    wait_vmcnt<0>();
  __syncthreads();
  load_frags(0, fa0, fb0);

  // KT is even for every supported shape (H and Im are multiples of 128,
  // BK <= 64); two k-tiles per trip keep the fragment sets in fixed registers.
  for (int kt = 0; kt < KT; kt += 2) {
    if (kt + C::STAGES - 1 < KT) issue(kt + C::STAGES - 1, (kt + C::STAGES - 1) % C::STAGES);
    load_frags(kt + 1, fa1, fb1);
    mfmas(fa0, fb0);
    sync_end(kt);
    if (kt + C::STAGES < KT) issue(kt + C::STAGES, (kt + C::STAGES) % C::STAGES);
    load_frags(kt + 2, fa0, fb0);
    mfmas(fa1, fb1);
    sync_end(kt + 1);
  }

  const int ldc = (C::MODE == kW13) ? mu * Im : H;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = ti.m0 + wm * C::TM + 16 * i + 4 * (lane >> 4) + r;
      if (p >= ti.seg_end) continue;
      uint16_t* crow = Cout + (size_t)p * ldc;
      if (C::MODE == kW13) {
#pragma unroll
        for (int j = 0; j < C::FN / 2; ++j) {
          const float g = acc[i][j][r], u = acc[i][j + C::FN / 2][r];
          crow[micro * Im + n0 + wn * (C::TN / 2) + 16 * j + fr] = float_to_bf16_bits(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          crow[n0 + wn * C::TN + 16 * j + fr] = float_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

inline long long max_m_tiles(long long R, int E, int bm) {
  const long long a = (R + (long long)E * (bm - 1)) / bm;
  return a < 1 ? 1 : a;
}

template <class C>
hipError_t launch_split(const void* a, const int32_t* perm, const int32_t* offsets, const void* b,
                        void* c, int T, int H, int E, int k, int Im, int mu, hipStream_t st) {
  const int n_tiles = (C::MODE == kW13) ? mu * (Im / C::HCOLS) : H / C::BN;
  const long long tiles = max_m_tiles((long long)T * k, E, C::BM) * n_tiles;
  const unsigned grid = (unsigned)((tiles + kXcds - 1) / kXcds * kXcds);
  hipLaunchKernelGGL(grouped_gemm_split<C>, dim3(grid), dim3(C::NTHR), 0, st, (const uint16_t*)a,
                     perm, offsets, (const uint16_t*)b, (uint16_t*)c, H, E, k, Im, mu, n_tiles);
  return hipGetLastError();
}

template <class C, bool DB = false, bool M32 = false>
hipError_t launch(const void* a, const int32_t* perm, const int32_t* offsets, const void* b,
                  void* c, int T, int H, int E, int k, int Im, int mu, hipStream_t st) {
  const int n_tiles = (C::MODE == kW13) ? mu * (Im / C::HCOLS) : H / C::BN;
  const long long tiles = max_m_tiles((long long)T * k, E, C::BM) * n_tiles;
  const unsigned grid = (unsigned)((tiles + kXcds - 1) / kXcds * kXcds);
  if constexpr (M32)
    hipLaunchKernelGGL(grouped_gemm32<C>, dim3(grid), dim3(C::NTHR), 0, st,
                       (const uint16_t*)a, perm, offsets, (const uint16_t*)b, (uint16_t*)c, H, E, k,
                       Im, mu, n_tiles);
  else if constexpr (DB)
    hipLaunchKernelGGL(grouped_gemm_db<C>, dim3(grid), dim3(C::NTHR), 0, st,
                       (const uint16_t*)a, perm, offsets, (const uint16_t*)b, (uint16_t*)c, H, E, k,
                       Im, mu, n_tiles);
  else
  hipLaunchKernelGGL(grouped_gemm<C>, dim3(grid), dim3(C::NTHR), 0, st,
                     (const uint16_t*)a, perm, offsets, (const uint16_t*)b, (uint16_t*)c, H, E, k,
                     Im, mu, n_tiles);
  return hipGetLastError();
}

}  // namespace fast
}  // namespace moe
