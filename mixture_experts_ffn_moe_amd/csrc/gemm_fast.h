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
//     tiles (v_mfma_f32_16x16x32_bf16); two waves per SIMD, so a wave's
//     accumulators and fragments share 256 registers.
#pragma once

#include "moe_common.h"

namespace moe {
namespace fast {

enum Mode { kW13 = 0, kDown = 1 };

typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int MODE_, int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_, int SB_ = STAGES_>
struct Cfg {
  static constexpr int MODE = MODE_, BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  // ring slots of the B (weight) tiles; A keeps STAGES.  SB = STAGES + 1 gives
  // the HBM-streamed weights one more k-tile of lead than the gathered rows.
  static constexpr int SB = SB_;
  // two row slots: the waits in the k loop count only weight copies as
  // possibly in flight, which the skipped row copies of short tiles rely on
  static_assert(STAGES == 2 && (SB == 2 || SB == 3), "ring depths");
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
  static constexpr int LDS_BYTES = (STAGES * BM + SB * BN) * BK * 2;
  static constexpr int HCOLS = (MODE == kW13) ? BN / 2 : BN;  // output columns per tile
  // h leaves the w13 GEMM rounded to bf16 (the down GEMM's MFMA operand); y
  // leaves block-scaled half, one block of kYBlock columns per tile row
  static_assert(MODE == kW13 || BN == kYBlock, "one y block per tile row");
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

// Workgroup barrier for the k loop.  __syncthreads() carries a memory fence
// that waits for every outstanding global load, including the direct-to-LDS
// copies still in flight for later k-tiles; this one waits only for the
// wave's LDS reads (so the slot they read may be refilled) and the copies the
// caller has already waited for.  The scheduling barriers keep the compiler
// from moving work across it.
__device__ __forceinline__ void kloop_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct Tile {
  int e, m0, seg_end, nt, valid;
};

// An optional dense segment run in the same launch after the routed tiles
// (the shared expert: every token in order, its own weights and output):
// A rows a[p] for p < rows (row stride H in w13 mode, w in down mode), B the
// segment's weights (w13: [2w, H], gate rows then up rows; down: [H, w]), C
// its output (w13: [rows, w]; down: [rows, H]).  rows == 0: none.
struct Extra {
  const uint16_t* a;
  const uint16_t* b;
  void* c;  // bf16 in w13 mode, block-scaled half of `rows` rows in down mode
  int rows, w;
};

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

// Logical tile of this workgroup (expert-major, then n-tile, then m-tile),
// decoded from the device-side offsets; XCD-aware: XCD x (= blockIdx % 8)
// takes the contiguous logical range [x*per, (x+1)*per).  offsets == nullptr
// is one dense segment of dense_rows rows (E = 1: the shared expert).
template <int BM>
__device__ __forceinline__ Tile decode(const int32_t* __restrict__ offsets, int E, int n_tiles,
                                       int dense_rows) {
  __shared__ int s_info[5];
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int off = 0, cnt = 0;
    if (offsets == nullptr) {
      cnt = lane == 0 ? dense_rows : 0;
    } else if (lane < E) {
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

// Wave-local tile decode: every wave computes the same result from the
// offsets with its own 64-lane scan, so no LDS slot or barrier is needed.
// An expert with cnt rows gets mt = ceil(cnt / BM) m-tiles of equal height
// (ceil(cnt / mt) rounded up to 16 rows, the last one shorter); t.seg_end is
// the end of this tile's rows.  Equal tiles take equal time, so the m-tiles
// that share an n-tile of weights run side by side and share it in L2.
// offsets == nullptr is one dense segment of dense_rows rows, as in decode().
template <int BM, bool EQ = true, bool XS = false>
__device__ __forceinline__ Tile decode_wave(const int32_t* __restrict__ offsets, int E, int n_tiles,
                                            int dense_rows, int x_rows = 0, int x_ntiles = 0) {
  const int lane = threadIdx.x & 63;
  int off = 0, cnt = 0;
  if (offsets == nullptr) {
    cnt = lane == 0 ? dense_rows : 0;
  } else if (lane < E) {
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
  // the extra dense segment's tiles follow the routed ones (expert index E)
  const int x_mt = XS ? (x_rows + BM - 1) / BM : 0;
  const int all = XS ? total + x_mt * x_ntiles : total;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int per = (all + kXcds - 1) / kXcds;
  const int L = xcd * per + slot;
  const bool ok = slot < per && L < all;
  const bool xt = XS && L >= total;
  const uint64_t hit = __ballot(lane < E && incl > L);
  const int e = ok && hit ? (__ffsll((long long)hit) - 1) : 0;
  const int e_incl = __shfl(incl, e), e_tiles = __shfl(tiles, e), e_mt = __shfl(mt, e);
  const int e_off = __shfl(off, e), e_cnt = __shfl(cnt, e);
  Tile t;
  t.valid = (ok && (hit || xt)) ? 1 : 0;
  const int local = xt ? L - total : L - (e_incl - e_tiles);
  const int s_mt = xt ? x_mt : e_mt, s_off = xt ? 0 : e_off, s_cnt = xt ? x_rows : e_cnt;
  const int mt_safe = s_mt > 0 ? s_mt : 1;
  const int rows = EQ ? (((s_cnt + mt_safe - 1) / mt_safe + 15) & ~15) : BM;  // <= BM
  t.e = xt ? E : e;
  t.m0 = s_off + (t.valid ? (local % mt_safe) * rows : 0);
  t.seg_end = min(t.m0 + rows, s_off + s_cnt);
  t.nt = t.valid ? local / mt_safe : 0;
  t.valid = __builtin_amdgcn_readfirstlane(t.valid);
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
  t.seg_end = __builtin_amdgcn_readfirstlane(t.seg_end);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  return t;
}

template <class C, bool PART = true, bool EQ = true, bool XS = false>
__global__ __launch_bounds__(C::NTHR, 1) void grouped_gemm(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B, void* __restrict__ Cout,
    int H, int E, int k, int Im, int mu, int n_tiles, int dense_rows, Extra ex) {
  // A ring (STAGES slots of BM x BK) followed by the B ring (SB slots of BN x BK)
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(C::STAGES * C::BM + C::SB * C::BN) * C::BK];

  // XS: the launch has an extra dense segment (a separate instantiation, so
  // the routed-only kernel carries none of its tile logic)
  const int x_ntiles = XS ? ((C::MODE == kW13) ? ex.w / C::HCOLS : (H + C::BN - 1) / C::BN) : 0;
  const Tile ti = decode_wave<C::BM, EQ, XS>(offsets, E, n_tiles, dense_rows, ex.rows, x_ntiles);
  if (!ti.valid) return;
  // a tile of the extra dense segment: its own A, B, C and width, one micro
  const bool xt = XS && ti.e == E;
  if (xt) {
    A = ex.a;
    B = ex.b;
    Cout = ex.c;
    Im = ex.w;
    mu = 1;
  }

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
    // A row: x row of route perm[p] (w13), row p of h (down: no perm is
    // passed, and none is read); a dense segment (no offsets, or the extra
    // segment) reads row p
    uint32_t r;
    if constexpr (C::MODE == kW13) {
      const uint32_t xr = (offsets == nullptr || xt) ? (uint32_t)p : (uint32_t)(perm[p] / k);
      r = xr * (uint32_t)H;
    } else {
      r = (uint32_t)p * (uint32_t)lda;
    }
    a_off[i] = (r + c * 8) * 2u;
  }
  const uint16_t* b_base;
  uint32_t b_ld;
  const int eb = xt ? 0 : ti.e;  // expert block of the weights
  if (C::MODE == kW13) {
    b_base = B + (size_t)(micro * E + eb) * (2 * Im) * H;
    b_ld = H;
  } else {
    b_base = B + ((size_t)eb * H + n0) * Im;
    b_ld = Im;
  }
  uint32_t b_off[C::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::B_PER_WAVE; ++i) {
    const int row = (wave + C::NW * i) * C::RPI + lrow;
    const int c = lpos ^ swz<C::CPR>(row);
    int wrow = row;
    if (C::MODE == kW13) wrow = row < C::BN / 2 ? n0 + row : Im + n0 + (row - C::BN / 2);
    // down: the last n-tile may reach past H (H % BN != 0); its rows past H
    // copy row H - 1 again, whose output columns are never stored (and, being
    // a copy of a stored column, leave the row's block maximum unchanged)
    else wrow = min(row, H - 1 - n0);
    b_off[i] = ((uint32_t)wrow * b_ld + c * 8) * 2u;
  }
  constexpr int A_SLOT = C::BM * C::BK, B_SLOT = C::BN * C::BK;  // elements
  const uint32_t ldsA = (uint32_t)(uintptr_t)smem;
  const uint32_t ldsB = ldsA + (uint32_t)(C::STAGES * A_SLOT) * 2u;

  // Row groups past the tile's rows (rounded up to the 16-row MFMA
  // fragments) are never read: their copies are skipped.  The waits below
  // only ever leave weight copies in flight, so they hold with any number of
  // row copies.
  const int a_rows = PART ? __builtin_amdgcn_readfirstlane(min(C::BM, (ti.seg_end - ti.m0 + 15) & ~15)) : C::BM;
  auto issue_a = [&](int kt) {
    const uint32_t sb = ldsA + (uint32_t)((kt % C::STAGES) * A_SLOT) * 2u;
    const uint16_t* abase = A + kt * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i)
      if ((wave + C::NW * i) * C::RPI < a_rows)
        dma16(sb + (uint32_t)((wave + C::NW * i) * C::RPI * C::BK) * 2u, abase, a_off[i]);
  };
  auto issue_b = [&](int kt) {
    const int kg = kt * C::BK;
    const uint32_t sb = ldsB + (uint32_t)((kt % C::SB) * B_SLOT) * 2u;
    const uint16_t* bbase = b_base + kg;
    if (C::MODE == kDown) {
      const int mm = kg / Im;
      bbase = b_base + (size_t)mm * E * H * Im + (kg - mm * Im);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i)
      dma16(sb + (uint32_t)((wave + C::NW * i) * C::RPI * C::BK) * 2u, bbase, b_off[i]);
  };

  // ---- MFMA fragment addressing (row = 16-aligned base + lane%16)
  // wave w runs on SIMD w % 4; with wm = w / WN each SIMD holds waves of
  // different row blocks, so the MFMA work skipped below for rows past the
  // expert's segment is taken off every SIMD alike
  const int wm = PART ? wave / C::WN : wave % C::WM;
  const int wn = PART ? wave % C::WN : wave / C::WM;
  // 16-row fragments of this wave that hold at least one row of the segment
  int nf = C::FM;
  if (PART) {
    const int rows = ti.seg_end - ti.m0 - wm * C::TM;
    nf = __builtin_amdgcn_readfirstlane(rows <= 0 ? 0 : min(C::FM, (rows + 15) / 16));
  }
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

  // Prologue.  Equal rings: A(s), B(s) for s < STAGES - 1.  SB = 3: B(0),
  // A(0), B(1), so that waiting for A(kt) leaves only B(kt+1) in flight.
  if (C::SB == C::STAGES) {
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s)
      if (s < KT) {
        issue_a(s);
        issue_b(s);
      }
  } else {
    issue_b(0);
    issue_a(0);
    if (1 < KT) issue_b(1);
  }

  // k loop; FULL: all FM fragments of this wave hold rows of the segment,
  // else only the first nf (possibly none: the wave then only copies and
  // waits).  The two variants are separate loops so that each keeps its
  // own register allocation.
  auto kloop = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    for (int kt = 0; kt < KT; ++kt) {
      // A(kt) and B(kt) have landed (this wave's copies; the barrier makes
      // every wave's visible); the slots refilled below were last read in
      // iteration kt - 1
      if (C::SB == C::STAGES) {
        if (kt + C::STAGES - 2 < KT)
          wait_vmcnt<(C::STAGES - 2) * C::NI>();
        else
          wait_vmcnt<0>();
        kloop_barrier();
        if (kt + C::STAGES - 1 < KT) {
          issue_a(kt + C::STAGES - 1);
          issue_b(kt + C::STAGES - 1);
        }
      } else {
        if (kt + 1 < KT)
          wait_vmcnt<C::B_PER_WAVE>();  // B(kt+1) may stay in flight
        else
          wait_vmcnt<0>();
        kloop_barrier();
        if (kt + 1 < KT) issue_a(kt + 1);
        if (kt + 2 < KT) issue_b(kt + 2);
      }
      const uint16_t* s = smem + (kt % C::STAGES) * A_SLOT;
      const uint16_t* sbt = smem + C::STAGES * A_SLOT + (kt % C::SB) * B_SLOT;
      if (FULL) {
#pragma unroll
        for (int ks = 0; ks < C::BK / 32; ++ks) {
          const int ch = ((ks * 4 + (lane >> 4)) ^ sw) * 8;
          bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
          for (int f = 0; f < C::FM; ++f) af[f] = *reinterpret_cast<const bf16x8*>(s + fa[f] + ch);
#pragma unroll
          for (int f = 0; f < C::FN; ++f) bfr[f] = *reinterpret_cast<const bf16x8*>(sbt + fb[f] + ch);
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
      } else if (nf > 0) {
#pragma unroll
        for (int ks = 0; ks < C::BK / 32; ++ks) {
          const int ch = ((ks * 4 + (lane >> 4)) ^ sw) * 8;
          bf16x8 bfr[C::FN];
#pragma unroll
          for (int f = 0; f < C::FN; ++f) bfr[f] = *reinterpret_cast<const bf16x8*>(sbt + fb[f] + ch);
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            if (i < nf) {
              const bf16x8 af = *reinterpret_cast<const bf16x8*>(s + fa[i] + ch);
#pragma unroll
              for (int j = 0; j < C::FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af, acc[i][j], 0, 0, 0);
            }
          }
        }
      }
    }
  };
  if (nf == C::FM)
    kloop(BoolTag<true>{});
  else
    kloop(BoolTag<false>{});

  // ---- epilogue.  The weights are the MFMA's first operand, so in block
  // (i, j) lane holds token row 16*i + lane%16 and the four consecutive
  // output columns 16*j + 4*(lane/16) + r, r = 0..3.  Stored straight from
  // there, every store instruction would write 32-byte pieces of 16 rows;
  // instead the tile goes through LDS (the ring is free once every wave has
  // passed the barrier) and leaves as whole 128-byte lines, 16 bytes per lane
  // (the down GEMM, whose tiles are short in K, ran 8% faster so).
  constexpr int OC = (C::MODE == kW13) ? C::HCOLS : C::BN;  // output columns of the tile
  constexpr int OB = 2;             // bf16 h, or the fp16 values of y
  constexpr int OS = OC * OB + 16;  // LDS row stride in bytes: rows 4 banks apart
  // the whole tile in one pass when it fits the ring, else one wave-row block
  // (TM rows) per pass
  constexpr int PASSES = (C::BM * OS <= C::LDS_BYTES) ? 1 : C::WM;
  constexpr int PROWS = C::BM / PASSES;
  static_assert(PROWS * OS <= C::LDS_BYTES, "output rows of a pass fit the ring");
  constexpr int LPR = OC * OB / 16, RPW = kWave / LPR;  // lanes per row, rows per store
  static_assert(LPR <= kWave && kWave % LPR == 0, "store lanes");
  const int ldc = (C::MODE == kW13) ? mu * Im : H;
  const int cq = 4 * (lane >> 4);
  const int rows = ti.seg_end - ti.m0;
  const int col0 = (C::MODE == kW13) ? micro * Im + n0 : n0;
  const int cb = (lane % LPR) * 16;
  char* so = reinterpret_cast<char*>(smem);

  // y (down): block-scaled half, one block = the tile row's BN columns.  A
  // row's block maximum: over the lane's values, across the four lanes that
  // share the row (lane ^ 16, lane ^ 32), then across the two waves that hold
  // its column halves (through LDS, past the staging area); the accumulators
  // are then scaled by 2^-e in registers and staged as fp16.
  if constexpr (C::MODE == kDown) {
    static_assert(C::WN == 2 && C::TN * 2 == C::BN, "two waves share a tile row");
    constexpr int MAX_OFF = C::LDS_BYTES - 2 * C::BM * 4;
    static_assert(MAX_OFF >= PROWS * OS, "row maxima past the staging rows");
    float* smax = reinterpret_cast<float*>(so + MAX_OFF);
    float rmax[C::FM];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(acc[i][j][r]));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      rmax[i] = m;
    }
    __syncthreads();  // every wave is past its last k-step: the ring is free
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) smax[wn * C::BM + wm * C::TM + 16 * i + lane] = rmax[i];
    }
    __syncthreads();
    const size_t out_rows = xt ? (size_t)ex.rows : (size_t)dense_rows * (size_t)k;
    int8_t* ye = reinterpret_cast<int8_t*>(reinterpret_cast<char*>(Cout) + out_rows * (size_t)ldc * 2);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int tr = wm * C::TM + 16 * i + (lane & 15);  // tile row
      const int e = yexp_of(fmaxf(rmax[i], smax[(1 - wn) * C::BM + tr]));
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = ldexpf(acc[i][j][r], -e);
      if (wn == 0 && lane < 16 && tr < rows)
        ye[(size_t)(ti.m0 + tr) * (size_t)((ldc + kYBlock - 1) / kYBlock) + col0 / kYBlock] = (int8_t)e;
    }
  }

#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    __syncthreads();
    if (PASSES == 1 || wm == pass) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int rt = wm * C::TM + 16 * i + (lane & 15) - pass * PROWS;  // row in this pass
        if (C::MODE == kW13) {
#pragma unroll
          for (int j = 0; j < C::FN / 2; ++j) {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = silu_f32(acc[i][j][r]) * acc[i][j + C::FN / 2][r];
            *reinterpret_cast<uint2*>(so + rt * OS + (wn * (C::TN / 2) + 16 * j + cq) * 2) = pack_bf16x4(v);
          }
        } else {
          typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            f16x4 hv;
#pragma unroll
            for (int r = 0; r < 4; ++r) hv[r] = (_Float16)acc[i][j][r];
            *reinterpret_cast<f16x4*>(so + rt * OS + (wn * C::TN + 16 * j + cq) * 2) = hv;
          }
        }
      }
    }
    __syncthreads();
    const int prow_end = min(rows - pass * PROWS, PROWS);
    for (int r0 = wave * RPW; r0 < prow_end; r0 += C::NW * RPW) {
      const int rr = r0 + lane / LPR;
      // down: columns past H (a partial last n-tile) are not stored
      if (rr < prow_end && (C::MODE == kW13 || col0 + cb / OB < ldc)) {
        const uint4 v = *reinterpret_cast<const uint4*>(so + rr * OS + cb);
        const size_t row = (size_t)(ti.m0 + pass * PROWS + rr);
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Cout) + (row * ldc + col0) * OB + cb) = v;
      }
    }
  }
}

inline long long max_m_tiles(long long R, int E, int bm) {
  const long long a = (R + (long long)E * (bm - 1)) / bm;
  return a < 1 ? 1 : a;
}

// offsets == nullptr: one dense segment of the T rows (E = k = mu = 1, the
// shared expert), A rows read in order.  ex: an extra dense segment run
// after the routed tiles in the same launch (ex.rows == 0: none).
template <class C, bool PART = true, bool EQ = true>
hipError_t launch(const void* a, const int32_t* perm, const int32_t* offsets, const void* b,
                  void* c, int T, int H, int E, int k, int Im, int mu, hipStream_t st,
                  Extra ex = Extra{nullptr, nullptr, nullptr, 0, 0}) {
  const int n_tiles = (C::MODE == kW13) ? mu * (Im / C::HCOLS) : (H + C::BN - 1) / C::BN;
  const int x_ntiles = (C::MODE == kW13) ? ex.w / C::HCOLS : (H + C::BN - 1) / C::BN;
  const long long tiles = max_m_tiles((long long)T * k, E, C::BM) * n_tiles +
                          (long long)((ex.rows + C::BM - 1) / C::BM) * x_ntiles;
  const unsigned grid = (unsigned)((tiles + kXcds - 1) / kXcds * kXcds);
  if (ex.rows > 0)
    hipLaunchKernelGGL((grouped_gemm<C, PART, EQ, true>), dim3(grid), dim3(C::NTHR), 0, st,
                       (const uint16_t*)a, perm, offsets, (const uint16_t*)b, c, H, E, k,
                       Im, mu, n_tiles, T, ex);
  else
    hipLaunchKernelGGL((grouped_gemm<C, PART, EQ, false>), dim3(grid), dim3(C::NTHR), 0, st,
                       (const uint16_t*)a, perm, offsets, (const uint16_t*)b, c, H, E, k,
                       Im, mu, n_tiles, T, ex);
  return hipGetLastError();
}

}  // namespace fast
}  // namespace moe
