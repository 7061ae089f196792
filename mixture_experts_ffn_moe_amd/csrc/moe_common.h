// Shared device helpers and the internal launcher interface of the MoE
// kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 64;  // one lane per expert in the top-k wave
constexpr int kXcds = 8;         // MI355X: 8 accelerator dies, 32 CUs each

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four fp32 values to four bf16 (round to nearest even) in 8 bytes, on the
// gfx950 packed conversion instruction.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 pack_bf16x4(f32x4 v) {
  const bf16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// SiLU(z) = z / (1 + e^-z), with the device's fast exponential and
// reciprocal (a few ulp in fp32, far below the bf16 rounding that follows;
// z -> -inf gives -0, z -> +inf gives z).
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
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
// and barrier themselves before reading the destination.  lds and sbase must
// be wave-uniform (scalar registers).
// m0 is a reserved register (the compiler sets it right before each of its
// own uses and keeps no value in it), so naming it as clobbered only states
// what the asm does; clang warns that the clobber of a reserved register is
// informational, which is silenced for this one statement.
__device__ __forceinline__ void dma16(uint32_t lds, const void* sbase, uint32_t voff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
#pragma clang diagnostic pop
}

// A pointer the caller knows to be wave-uniform, moved to scalar registers
// (lane 0's value).  readfirstlane takes and returns int: each 32-bit half is
// taken back to uint32_t before it is widened, so the low half is
// zero-extended (a sign-extended low half with bit 31 set would turn the
// address into 0xffffffff........).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// Orderable 32-bit key of a float: unsigned order equals numeric order and
// -0.0 maps to the key of +0.0; every finite float's key is nonzero.
__device__ __forceinline__ uint32_t orderable(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Maximum of v over the 64 lanes, returned to every lane.  DPP row shifts
// build the maximum of each 16-lane row in its lane 15, row broadcasts carry
// it into lane 63; a lane whose DPP source is out of range or masked keeps its
// own value (old = v), which max leaves unchanged.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xf, false);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8
  v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// y, the down projection's output handed to the finalize, in the bf16 layers:
// "block-scaled half".  Each row is cut into blocks of kYBlock columns; a
// block stores its values as fp16 scaled by a power of two chosen from the
// block's largest magnitude M (the values times 2^-e land in (-2^15, 2^15)
// and round to at most 2^15, well within fp16's range), and e as one int8.  So y keeps 11 significant bits
// (bf16 has 8) in the bytes of bf16 plus one per block: a bf16 y would be a
// third rounding between the accumulator and the output, enough at outputs of
// magnitude 4 and more to pass the bf16 bar of 2e-2.  Layout of a y buffer of
// `rows` rows and H columns: values fp16 [rows, H], then exponents int8
// [rows, ceil(H / kYBlock)] (a partial last block when H % kYBlock != 0);
// y[p][n] = values[p][n] * 2^exponents[p][n / kYBlock].
constexpr int kYBlock = 256;
inline size_t y_half_bytes(long long rows, int H) {
  return (size_t)rows * H * 2 + (size_t)rows * ((H + kYBlock - 1) / kYBlock);
}
// e for a block whose largest magnitude is M: floor(log2 M) - 14, clamped to
// int8 (0 for M = 0; blocks below 2^-114 lose only digits far below any bar).
__device__ __forceinline__ int yexp_of(float M) {
  if (!(M > 0.0f)) return 0;
  int e2;
  (void)frexpf(M, &e2);  // M = f * 2^e2, f in [0.5, 1): floor(log2 M) = e2 - 1
  const int e = e2 - 15;
  return e < -128 ? -128 : (e > 127 ? 127 : e);
}

// Element loads/stores for the two supported element types.  bf16 tensors
// are moved as raw 16-bit patterns.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_float(*p); }
  static __device__ __forceinline__ float to_f(uint16_t v) { return bf16_bits_to_float(v); }
  static __device__ __forceinline__ uint16_t from_f(float v) { return float_to_bf16_bits(v); }
};

// ---------------------------------------------------------------------------
// Launchers (host side).  Shapes are validated by the caller; every launcher
// only enqueues on `stream` and returns the launch status.

struct Shape {
  int T, H, E, k, Im, mu;
  bool bf16;
  bool renorm;  // routing weights renormalised over the k selected experts
  long long R() const { return (long long)T * k; }
};

// Tokens per router workgroup; with a non-null `hist` the router also writes
// hist[b][e] (int32, kMaxExperts per row) = routes of tokens
// [kRouteTokTile*b, kRouteTokTile*(b+1)) that went to expert e.
constexpr int kRouteTokTile = 16;
inline size_t route_hist_bytes(const Shape& s) {
  return (size_t)((s.T + kRouteTokTile - 1) / kRouteTokTile) * kMaxExperts * 4;
}

hipError_t launch_route(const Shape& s, const void* x, const float* wg, const float* bias,
                        float* logits, int32_t* ids, float* w, hipStream_t st,
                        int32_t* hist = nullptr);

hipError_t launch_permute(const Shape& s, const int32_t* ids, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t st);

// Same outputs as launch_permute from the router's per-block histograms.
hipError_t launch_permute_hist(const Shape& s, const int32_t* ids, const int32_t* hist,
                               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                               hipStream_t st);

hipError_t launch_gather(const Shape& s, const void* x, const int32_t* perm, void* xp,
                         hipStream_t st);

hipError_t launch_w13_swiglu(const Shape& s, const void* x, const int32_t* perm,
                             const int32_t* offsets, const void* w1, void* h, hipStream_t st);

hipError_t launch_down(const Shape& s, const void* h, const int32_t* offsets, const void* w2,
                       void* y, hipStream_t st);
// bf16 only: the routed grouped GEMM and one dense segment of the T tokens in
// order (the shared expert: weights w1d [2*wd, H] / w2d [H, wd], outputs
// hd [T, wd] / yd [T, H]) in one launch.
hipError_t launch_w13_swiglu_with_dense(const Shape& s, const void* x, const int32_t* perm,
                                        const int32_t* offsets, const void* w1, void* h,
                                        const void* w1d, void* hd, int wd, hipStream_t st);
hipError_t launch_down_with_dense(const Shape& s, const void* h, const int32_t* offsets,
                                  const void* w2, void* y, const void* hd, const void* w2d,
                                  void* yd, int wd, hipStream_t st);

// ys: the shared expert's output [T, H] added after the routed sum, or nullptr.
hipError_t launch_finalize(const Shape& s, const void* y, const int32_t* inv, const float* w,
                           void* out, hipStream_t st, const void* ys = nullptr);

// Small-token path (decode.hip).
size_t decode_scratch_bytes();
bool decode_supported(const Shape& s);
// Shared expert of the small-token path: gate|up weights w1 [2*Is, H], down
// weights w2 [H, Is], its SwiGLU activations written to h [T, Is].
struct SharedExpert {
  const void* w1;
  const void* w2;
  int Is;
  void* h;
};
bool decode_shared_supported(int Is);
hipError_t launch_decode(const Shape& s, const void* x, const float* wg, const float* bias,
                         const void* w1, const void* w2, void* out, float* logits, int32_t* ids,
                         float* w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                         void* h, void* scratch, hipStream_t st,
                         const SharedExpert* shared = nullptr);

}  // namespace moe
