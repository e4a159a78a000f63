// far_kernels.hpp -- HIP kernels of the fused "sum of partials + residual add + RMSNorm
// (+ fp8 quant)" epilogue, written for gfx950 (CDNA4, wave64).
//
// The operation is defined on page "vllm.models.common.ops.fused_allreduce_rms_norm"
// (fused_allreduce_rms_norm: (normed_output, new_residual) = norm(all_reduce(partials),
// residual), accumulation wider than the storage type, weight_bias + gamma) and page
// "vllm.compilation.fusion"
// (kFp8StaticTensorSym / kFp8DynamicTokenSym epilogues).
//
// The path moves ~(P + 3) * 2 bytes per element for ~(P + 4) flops, far below the
// fp32 ridge of the chip, so everything here is about HBM streaming: 128-bit loads
// that make each wave instruction read 1 KiB of contiguous row, a window of a lane's
// loads kept in flight ahead of their use, the new residual row kept in registers (no
// second pass through memory), and one wave or LDS reduction per row. No MFMA: this is
// not a contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace far {

constexpr int kMaxPartials = 8;
constexpr int kWave = 64;
constexpr int kMaxWavesPerBlock = 16;
constexpr int kMaxPacksPerLane = 5;
constexpr uint32_t kXcds = 8;  // accelerator complex dies of the part, each with its own L2
constexpr float kE4m3Max = 448.0f;

enum Quant : int {
  kQuantNone = 0,
  kQuantStatic = 1,          // one static scale per tensor
  kQuantDynamic = 2,         // one dynamic scale per token
  kQuantDynamicGroup = 3,    // one dynamic scale per kFp8Group elements of a row
  kQuantDynamicTensor = 4,   // one dynamic scale per tensor (second and third kernels)
};
constexpr int kFp8Group = 128;

// 16-byte loads each lane keeps in flight while summing. Only one pack's accumulators
// are live at a time (the sum is pack-major), so the window is bounded by what the
// finished packs' x * w values leave of the 128-VGPR budget; the values here keep
// every instantiation within it without spilling (the build checks). Measured on
// prefill shapes: at five packs with P <= 4 a window of 9 is 2% faster than 6; at four
// packs with 2 <= P <= 4 every load in flight (16 covers them) is up to 12% faster than
// 5 (P = 1 gains nothing); at three packs with P >= 5, 21 (all loads for P <= 6) gains
// up to 2% over 10. The binary64 accumulators of a pack (fp16) take 16 VGPRs: with
// P >= 7 their three-pack window is 18 (21 would spill).
template <int NPACK, int P, int QUANT, bool WIDE_SUM>
constexpr int load_window_whole() {
  return QUANT == kQuantDynamicGroup
             ? (NPACK <= 2 ? 12 : (NPACK == 3 ? 8 : 5))
             : (NPACK <= 2 ? 16
                : NPACK == 3 ? (P >= 7 && WIDE_SUM ? 18 : P >= 5 ? 21 : 10)
                : NPACK == 4 ? (P >= 2 && P <= 4 ? 16 : 5)
                             : (P <= 4 ? 9 : 6));
}
// Rows ending in a partial pack (RAGGED) load it ahead of the packs, in a window that
// many loads longer, where registers allow (the shallower lanes with fewer partials);
// elsewhere they load it after the packs, with the five-pack window two loads shorter.
template <int NPACK, int P, int QUANT>
constexpr bool tail_early() {
  return NPACK == 1 || (NPACK == 2 && P <= 6) || (NPACK == 3 && P <= 4) ||
         (NPACK == 4 && P <= 3 && QUANT != kQuantDynamicGroup);
}
template <int NPACK, int P, int QUANT, bool WIDE_SUM, bool RAGGED>
constexpr int load_window() {
  constexpr int w = load_window_whole<NPACK, P, QUANT, WIDE_SUM>();
  return !RAGGED ? w : tail_early<NPACK, P, QUANT>() ? w + P + 1 : NPACK == 5 ? w - 2 : w;
}

// Deepest decode launch (packs per lane) whose products x * w are pinned where they are
// computed (see far_vec_kernel).
constexpr int kPinXwMaxPacks = 2;

// Deepest launch (packs per lane) whose binary64-sum (fp16) kernel keeps x * w in
// registers rather than the packed new residual (see far_vec_kernel).
constexpr int kKeepXwMaxPacks = 2;

// Packs per lane a mode supports: the per-group epilogue needs a little more than the
// others, and at five packs it would spill.
constexpr int max_packs_for(int quant) { return quant == kQuantDynamicGroup ? 4 : kMaxPacksPerLane; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Everything a launch needs, passed by value in the kernel arguments (the partial
// pointers included, so no device-side pointer table is needed).
struct KernelArgs {
  const void* partials[kMaxPartials];
  const void* residual;   // may be null: no residual input
  const void* gamma;
  void* residual_out;     // may be null: new residual not written
  void* norm_out;         // may be null with quantisation
  uint8_t* quant_out;      // fp8 e4m3fn codes
  float* scale_out;        // dynamic scales: [T] per token, [T, groups] per group, [1] per tensor
  const float* scale;      // [1] static scale
  float* workspace;        // per-tensor mode: [2T] per-row max |y|, then per-row r
  int64_t num_tokens;
  int32_t hidden;
  int32_t num_partials;
  int32_t groups;          // ceil(hidden / kFp8Group)
  float eps;
  float weight_bias;
};

// binary32 value with the same rounding to fp16 as the binary64 v: v truncated to binary32,
// with the last bit set when the truncation dropped anything (round-to-odd), so the
// result is never a midpoint between two values of the coarser format.
__device__ __forceinline__ float round_odd_f32(double v) {
  const float r = static_cast<float>(v);  // nearest even
  const double back = static_cast<double>(r);
  uint32_t b = __float_as_uint(r);
  // inexact (NaN compares unequal to everything, and its conversion is already NaN):
  // step one unit toward zero if rounding went past v, then make the last bit odd
  const bool inexact = (back != v) & (v == v);
  const uint32_t past = __builtin_fabs(back) > __builtin_fabs(v) ? 1u : 0u;
  b = inexact ? ((b - past) | 1u) : b;
  return __uint_as_float(b);
}

// ---------------------------------------------------------------- storage formats
// Two storage values per 32-bit word; conversions to storage round to nearest even
// (gfx950 has a packed bf16 convert; fp16 converts honour the default RNE mode).
struct Bf16 {
  using Acc = f32x2;  // binary32 sum (see "the sum" below)
  using AccScalar = float;
  static __device__ __forceinline__ f32x2 unpack(uint32_t w) {
    f32x2 r;
    r.x = __uint_as_float(w << 16);
    r.y = __uint_as_float(w & 0xffff0000u);
    return r;
  }
  static __device__ __forceinline__ uint32_t pack(f32x2 v) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  static __device__ __forceinline__ float load1(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  static __device__ __forceinline__ float round1(float v) {
    f32x2 t = {v, 0.0f};
    return unpack(pack(t)).x;
  }
  static __device__ __forceinline__ void store1(void* p, int64_t i, float v) {
    f32x2 t = {v, 0.0f};
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(pack(t) & 0xffffu);
  }
  // two sums rounded to storage (one rounding each), and one sum as the binary32 value
  // that rounds to storage the same way
  static __device__ __forceinline__ uint32_t pack_sum(Acc s) { return pack(s); }
  static __device__ __forceinline__ float sum_to_f32(AccScalar s) { return s; }
};

struct Fp16 {
  using Acc = f64x2;  // exact binary64 sum (see "the sum" below)
  using AccScalar = double;
  static __device__ __forceinline__ f32x2 unpack(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  }
  static __device__ __forceinline__ uint32_t pack(f32x2 v) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float load1(const void* p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  }
  static __device__ __forceinline__ float round1(float v) {
    return static_cast<float>(static_cast<_Float16>(v));
  }
  static __device__ __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
  }
  static __device__ __forceinline__ uint32_t pack_sum(Acc s) {
    return pack(f32x2{round_odd_f32(s.x), round_odd_f32(s.y)});
  }
  static __device__ __forceinline__ float sum_to_f32(AccScalar s) { return round_odd_f32(s); }
};

// ---------------------------------------------------------------- the sum
// The new residual is the sum of the P partials and the residual, rounded once to the
// storage type (page "vllm.models.common.ops.fused_allreduce_rms_norm": accumulation
// wider than the storage type, fp32_acc=True). The terms are integer multiples of the
// quantum of the smallest one, so a binary32 sum is exact while every partial sum stays
// below 2^24 quanta: for P + 1 terms whose exponents lie within 16 - log2(P + 1) binades
// of each other for bf16 (8 significant bits; 12 binades at P = 8), but only within
// 13 - log2(P + 1) binades for fp16 (11 significant bits; 9 at P = 8), which ordinary
// data exceeds often enough that the binary32 sum of fp16 terms regularly lands on the
// other side of a rounding boundary. So bf16 terms are summed in binary32 (as the page
// accumulates) and fp16 terms in binary64, where the sum of up to nine of them is always
// exact (every fp16 value is a multiple of 2^-24 below 2^16). The binary64 sum is rounded
// to fp16 through binary32 with round-to-odd, which rounds exactly as a direct rounding
// would (binary32 carries more than two bits beyond fp16), then the hardware's
// round-to-nearest-even conversion.

// OCP fp8 e4m3fn code of v: NaN -> 0x7F with the sign kept; the magnitude is clamped
// to 448 and rounded to nearest even on the e4m3 grid (3 mantissa bits, exponent
// bias 7, subnormals k * 2^-9). Written from the format's definition with integer
// operations on the fp32 bits, so the result does not depend on a hardware mode.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag_bits = u & 0x7fffffffu;
  const float mag = fminf(__uint_as_float(mag_bits), kE4m3Max);  // +inf -> 448
  const uint32_t a = __float_as_uint(mag);
  // normal range (>= 2^-6): keep 3 of the 23 mantissa bits, round half to even on the
  // 20 dropped bits, then rebias the exponent from 127 to 7
  const uint32_t rounded = a + 0x7ffffu + ((a >> 20) & 1u);
  const uint32_t normal = (rounded >> 20) - (120u << 3);
  // subnormal range: the grid is k * 2^-9; scaling by 2^9 is exact and rint is RNE.
  // k == 8 is the smallest normal, whose code is also 8.
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(mag * 512.0f));
  uint32_t code = (a < 0x3c800000u) ? sub : normal;
  code = (mag_bits > 0x7f800000u) ? 0x7fu : code;
  return sign | code;
}

// Four e4m3 codes in one word, little-endian (element 0 in the low byte).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  return e4m3_code(a) | (e4m3_code(b) << 8) | (e4m3_code(c) << 16) | (e4m3_code(d) << 24);
}

// ---------------------------------------------------------------- wave reductions
// DPP butterfly inside each 16-lane row, then row broadcasts (GFX9 row_bcast15 /
// row_bcast31) fold the four rows into lane 63, which is read as a scalar.
__device__ __forceinline__ float wave_sum(float v) {
  int x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false)); // row_half_mirror
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false)); // row_mirror
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false)); // row_bcast15
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false)); // row_bcast31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Max of unsigned values (used on |y| bit patterns: for non-negative floats the bit
// pattern order is the value order, and NaN patterns sort above +inf, so the max
// propagates NaN).
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xA, 0xF, false)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xC, 0xF, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// ---------------------------------------------------------------- vector kernel
// One team of `waves_per_row` wavefronts per token row, `rows_per_block` teams per
// workgroup. Lane l of a team owns the 16-byte packs l + k * team_lanes, k < NPACK
// (8 storage elements each), and is the only lane that writes those elements, so
// residual_out may coincide with residual or a partial: every element is read before
// the lane that owns it writes it.
//
// Per element the kernel keeps xw = x * (weight_bias + gamma) in fp32 registers, where
// x is the rounded new residual. Then
//   norm_out = RNE(xw * r)                       r = 1 / sqrt(sum x^2 / H + eps)
//   static   : code = E4M3(xw * (r / S))         = E4M3(y / S)
//   dynamic  : scale = r * m / 448, code = E4M3(xw * (448 / m)),  m = max_h |xw|
// (r cancels from y / scale, so the dynamic codes need no second reduction: the
// row's max |y| is r * m because multiplying by r > 0 preserves order). The fp8
// conversion is gfx950's v_cvt_pk_fp8_f32 (round to nearest even, OCP e4m3) after a
// clamp to [-448, 448]. A row holding any non-finite value (NaN or inf in x * w, or a
// non-finite r or multiplier) takes an exact elementwise path instead, which maps NaN
// to the NaN code as the clamp cannot.
//
// Workgroups of up to 1024 lanes: the compiler then keeps each wave within 128 VGPRs,
// four waves per SIMD, which still leaves tens of KiB of loads in flight per CU.
constexpr int kVecMaxThreads = 1024;

__device__ __forceinline__ float clamp448(float v) {
  return __builtin_amdgcn_fmed3f(v, -kE4m3Max, kE4m3Max);
}

// Two fp8 codes of finite values (clamped first) in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3_pair_fast(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false)) & 0xffffu;
}

__device__ __forceinline__ bool finite_f32(float v) {
  return (__float_as_uint(v) & 0x7fffffffu) < 0x7f800000u;
}

// max |y| over a set of elements with y = xw * r, from m = max |xw| (as fp32 bits,
// NaN above inf) and the row's r >= 0: multiplying by r > 0 keeps the order, and the
// IEEE special cases (NaN, inf * 0, 0 * inf) follow the elementwise product.
__device__ __forceinline__ float amax_of(uint32_t m, float r) {
  if (m > 0x7f800000u || r != r || r == __builtin_inff()) return __builtin_nanf("");
  if (r == 0.0f) return (m == 0x7f800000u) ? __builtin_nanf("") : 0.0f;
  return r * __uint_as_float(m);
}

// dynamic scale from a max |y|: max / 448, 1.0 for an all-zero set, NaN stays NaN
__device__ __forceinline__ float scale_of(float amax) {
  return (amax == 0.0f) ? 1.0f : amax / kE4m3Max;
}

// max over the 16 lanes of a DPP row (the lanes holding one 128-element group)
__device__ __forceinline__ uint32_t row16_umax(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// The cross-wave step of a row: the team's waves w0 .. w0 + n - 1 have left their
// partial sums (and, when MAX, maxima) in slots of one parity's kMaxWavesPerBlock LDS
// slots. Lane i of every 16-lane DPP row reads slot i (one LDS read per array for all
// the slots, instead of one read per team wave, whose round trips would follow one
// another, or a loop over the team's lanes), slots outside the team count as 0, and four
// DPP steps inside the row combine the 16 values. The pairwise steps are symmetric, so
// every lane ends with the same total, and the order of the additions depends only on
// the slots, so results are reproducible.
static_assert(kMaxWavesPerBlock == 16, "one slot per lane of a 16-lane DPP row");

__device__ __forceinline__ float row16_sum(float v) {
  int x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false)); // row_half_mirror
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false)); // row_mirror
  return v;
}

// The slot a lane reads: its position in its 16-lane row, computed where it is used rather
// than hoisted out of a row loop (where it would hold a register through the whole loop).
__device__ __forceinline__ int slot_of_lane() {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0" : "=v"(lane));
  return lane & (kMaxWavesPerBlock - 1);
}

template <bool MAX>
__device__ __forceinline__ void team_reduce(const float* sum_slots, const uint32_t* max_slots, int w0,
                                            int n, float* total, uint32_t* m) {
  const int i = slot_of_lane();
  const bool mine = i >= w0 && i < w0 + n;
  const float s = sum_slots[i];
  uint32_t mx = 0u;
  if constexpr (MAX) mx = max_slots[i];
  *total = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                         __builtin_bit_cast(int, row16_sum(mine ? s : 0.0f))));
  if constexpr (MAX)
    *m = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(row16_umax(mine ? mx : 0u))));
}

// The max alone, the same way (the generic kernel takes it in a pass of its own).
__device__ __forceinline__ uint32_t team_umax(const uint32_t* slots, int w0, int n) {
  const int i = slot_of_lane();
  const uint32_t v = slots[i];
  return static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(row16_umax(i >= w0 && i < w0 + n ? v : 0u))));
}

// Eight codes of one pack: hardware conversion when `fast` (every value finite and
// the multiplier finite), else the exact software conversion of (xw * r) * (1 / d), with
// d = denom, or the dynamic scale of a max |y| of denom when DENOM_IS_AMAX; d and its
// reciprocal are taken only on that (rare) path.
__device__ __forceinline__ u32x2 pack_codes_fast(const float* xw, float mul) {
  u32x2 q;
  q.x = e4m3_pair_fast(xw[0] * mul, xw[1] * mul) | (e4m3_pair_fast(xw[2] * mul, xw[3] * mul) << 16);
  q.y = e4m3_pair_fast(xw[4] * mul, xw[5] * mul) | (e4m3_pair_fast(xw[6] * mul, xw[7] * mul) << 16);
  return q;
}

template <bool DENOM_IS_AMAX = false>
__device__ __forceinline__ u32x2 pack_codes_exact(const float* xw, float r, float denom) {
  // kept on this path: hoisted out of it, the divisions would run on every row
  float d = denom;
  asm volatile("" : "+v"(d));
  if constexpr (DENOM_IS_AMAX) d = scale_of(d);
  const float inv_y = 1.0f / d;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (xw[e] * r) * inv_y;
  u32x2 q;
  q.x = e4m3_pack4(y[0], y[1], y[2], y[3]);
  q.y = e4m3_pack4(y[4], y[5], y[6], y[7]);
  return q;
}

template <bool DENOM_IS_AMAX = false>
__device__ __forceinline__ u32x2 pack_codes(const float* xw, float mul, bool fast, float r,
                                            float denom) {
  // likely: the exact path's code goes after the loop, off the fast path's fetch
  if (__builtin_expect(fast, 1)) return pack_codes_fast(xw, mul);
  return pack_codes_exact<DENOM_IS_AMAX>(xw, r, denom);
}

// Buffer resource (V#) over `bytes` bytes at `base`: raw addressing (stride 0), so a
// load at a byte offset >= bytes returns zeros and a store there is dropped by the
// hardware range check. Every access is kept either wholly inside or wholly outside its
// range: 16-byte packs at pack-aligned offsets of ranges that are whole packs, and the
// narrower accesses of a row's partial last pack below.
constexpr int kRsrcWord3 = 0x00020000;  // GFX9 family: 32-bit data format, raw buffer
constexpr int kNonTemporal = 2;         // cache-policy bit: streamed once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t byte_off,
                                                           int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(base)) + byte_off, 0, bytes, kRsrcWord3);
}

// ---------------------------------------------------------------- partial last pack
// A row of H elements with H % 8 != 0 ends in a pack of n = H % 8 elements. Its lane
// moves them with narrower accesses, each either wholly inside the row or wholly
// outside it: 4-byte words for the element pairs, a 2-byte access for an odd last
// element (fp8 codes: 2-byte pairs and one byte). An access that is not wanted gets the
// offset `end` (the range's size), which the range check turns into a zero load or a
// dropped store.
struct TailAt {
  int pair[3];  // byte offsets of the element pairs 0-1, 2-3, 4-5
  int last;     // byte offset of element n - 1 when n is odd
  int last_dw;  // 32-bit word holding element n - 1 (low half) when n is odd
};

// The partial pack of a row of H elements, `elem` bytes each (2 for the storage type,
// 1 for the codes). H passes through an empty asm statement first, so the offsets are
// computed where they are used instead of being hoisted out of the row loop and held
// in scalar registers across it.
__device__ __forceinline__ TailAt tail_at(int H, int elem) {
  asm volatile("" : "+s"(H));
  const int at = (H >> 3) * 8 * elem;
  const int n = H & 7;
  const int end = H * elem;
  TailAt t;
#pragma unroll
  for (int d = 0; d < 3; ++d) t.pair[d] = (2 * d + 2 <= n) ? at + 2 * elem * d : end;
  t.last = (n & 1) ? at + elem * (n - 1) : end;
  t.last_dw = (n - 1) >> 1;
  return t;
}

// The same for one lane of a wave: lanes other than the pack's owner get the offset
// `end` everywhere, so their accesses fall outside the range (zeros, no memory
// request) and the whole wave can run the loads without a branch.
__device__ __forceinline__ TailAt tail_at_lane(int H, int elem, bool mine) {
  TailAt t = tail_at(H, elem);
  const int end = H * elem;
#pragma unroll
  for (int d = 0; d < 3; ++d) t.pair[d] = mine ? t.pair[d] : end;
  t.last = mine ? t.last : end;
  return t;
}

// The loads of the first n elements of a storage pack (POL: cache policy): the three
// element pairs, and in the fourth word the odd last element. Nothing here uses the
// loaded values, so the loads stay in flight until tail_merge.
template <int POL>
__device__ __forceinline__ u32x4 tail_load(__amdgpu_buffer_rsrc_t rsrc, const TailAt& t) {
  u32x4 v;
#pragma unroll
  for (int d = 0; d < 3; ++d) v[d] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, t.pair[d], 0, POL);
  v[3] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, t.last, 0, POL);
  return v;
}

// The pack from tail_load's words: the odd last element (zero when n is even) moves to
// the low half of its word, which was outside the row and read as zero; the elements
// past n are zero.
__device__ __forceinline__ u32x4 tail_merge(u32x4 v, int last_dw) {
  const uint32_t e = v[3];
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 3; ++d) r[d] = v[d] | (d == last_dw ? e : 0u);
  r[3] = last_dw == 3 ? e : 0u;
  return r;
}

template <int POL>
__device__ __forceinline__ void tail_store(u32x4 v, __amdgpu_buffer_rsrc_t rsrc, const TailAt& t) {
#pragma unroll
  for (int d = 0; d < 3; ++d) __builtin_amdgcn_raw_buffer_store_b32(v[d], rsrc, t.pair[d], 0, POL);
  uint32_t e = v[0];
#pragma unroll
  for (int d = 1; d < 4; ++d) e = (d == t.last_dw) ? v[d] : e;
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(e), rsrc, t.last, 0, POL);
}

// the first n codes of a pack's eight (element i in byte i of q)
template <int POL>
__device__ __forceinline__ void tail_store_codes(u32x2 q, __amdgpu_buffer_rsrc_t rsrc,
                                                 const TailAt& t) {
  const uint32_t half[3] = {q.x, q.x >> 16, q.y};
#pragma unroll
  for (int d = 0; d < 3; ++d)
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(half[d]), rsrc, t.pair[d], 0, POL);
  // odd n: code n - 1 is byte 2 * last_dw of the pack
  const uint32_t word = t.last_dw < 2 ? q.x : q.y;
  const uint32_t byte = word >> (16 * (t.last_dw & 1));
  __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(byte), rsrc, t.last, 0, POL);
}

// Offset given to the 16-byte accesses of a row's partial last pack: past the end of
// any row range (and, halved, of any code range), and unique to that pack's slot.
constexpr int kTailOff = 0x7ffffff0;

// CACHED_RESIDUAL: the new residual is stored with the default cache policy (written
// back later) instead of streamed out; measured faster on prefill-sized batches and
// slower on decode-sized ones, whose kernels end with the write-back.
template <typename Fmt, int P, int NPACK, int QUANT, bool RAGGED, bool CACHED_RESIDUAL = false>
__global__ void __launch_bounds__(kVecMaxThreads)
far_vec_kernel(const KernelArgs a, const int waves_per_row, const int rows_per_block) {
  // reduction slots, double buffered by row-loop parity so that a wave starting the
  // next row cannot overwrite values another wave of its team is still reading
  __shared__ float red_sum[2][kMaxWavesPerBlock];
  __shared__ uint32_t red_max[2][kMaxWavesPerBlock];

  const int team_lanes = waves_per_row * kWave;
  const int tid = static_cast<int>(threadIdx.x);
  // A team is a whole number of waves, so the team (and the row) is uniform across a
  // wave: the row's buffer descriptors live in scalar registers and each lane adds a
  // 32-bit byte offset.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave / waves_per_row;
  const int lane = tid - team * team_lanes;
  const int H = a.hidden;
  const int row_bytes = H * 2;
  // RAGGED (H % 8 != 0): the lane that owns the partial last pack gives that slot's
  // 16-byte accesses the offset kTailOff, so they read zeros and their stores are
  // dropped, and moves the pack's n = H % 8 elements with the narrower accesses above
  // (the slot is recognised by that offset, so no other state is kept for it).
  int voff[NPACK];  // byte offset of each of this lane's packs inside a row (may be
                    // past the end: then loads read zeros and stores are dropped)
#pragma unroll
  for (int k = 0; k < NPACK; ++k) {
    voff[k] = (lane + k * team_lanes) * 16;
    if constexpr (RAGGED)
      if ((H & 7) != 0 && lane + k * team_lanes == (H >> 3)) voff[k] = kTailOff;
  }
  // the wave of the team that holds the partial pack (uniform across the wave)
  const bool tail_wave = RAGGED && (H & 7) != 0 &&
                         __builtin_amdgcn_readfirstlane(lane >> 6) == ((H >> 3) % team_lanes) >> 6;

  // ---- gamma: shared by every row, loaded once per team and kept in registers
  const __amdgpu_buffer_rsrc_t g_rsrc = row_rsrc(a.gamma, 0, row_bytes);
  u32x4 g[NPACK];
#pragma unroll
  for (int k = 0; k < NPACK; ++k) g[k] = __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, voff[k], 0, 0);
  if constexpr (RAGGED) {
#pragma unroll
    for (int k = 0; k < NPACK; ++k)
      if (voff[k] == kTailOff) g[k] = tail_merge(tail_load<0>(g_rsrc, tail_at(H, 2)), tail_at(H, 2).last_dw);
  }
  const float wb = a.weight_bias;

  // Grid-stride loop over rows: with fewer workgroups than row groups, a team starts
  // the loads of its next row right after the stores of the current one, so reads and
  // writes of different rows overlap. The loop bound is uniform across the workgroup
  // (every team takes the same number of trips, as the barriers require). Row indices
  // are 32-bit unsigned: T < 2^31 and a sweep adds fewer than 2^25 rows (at most 2^20
  // workgroups of at most 16 rows), so no index wraps, and the loop bound and the
  // team's row test are scalar compares (the scalar unit has no 64-bit ordered compare;
  // 64-bit indices put a vector compare ahead of every row's descriptors).
  const uint32_t num_rows = static_cast<uint32_t>(a.num_tokens);
  const uint32_t rows_per_sweep = gridDim.x * static_cast<uint32_t>(rows_per_block);
  // The static scale is read once, here, before the kernel's first store: the compiler
  // can then load it through the scalar cache while the first row loads. Read after a
  // row's stores, it became a vector load whose wait (the vector memory counter counts
  // stores too) also waited for those stores, on the row's critical path.
  float static_scale = 1.0f;
  if constexpr (QUANT == kQuantStatic) static_scale = a.scale[0];
  // Workgroups are dealt to the 8 XCDs in turn (workgroup b runs on XCD b % 8, each XCD
  // with its own L2). When the grid loops over the rows (fewer row slots than rows) and
  // is a multiple of 8, each XCD takes a contiguous block of the grid's logical blocks
  // instead, so that the rows one L2 serves are adjacent in memory: P = 2, 2048 x 5120
  // dynamic fp8 0.75% faster, at hidden 5124 1.6%. A grid of one row per slot keeps the
  // hardware order, in which the workgroups dispatched together cover adjacent rows:
  // remapped, P = 8, 16384 x 3584 was 6% slower and the decode batches 1-3% slower.
  // Either way a permutation of the blocks: every row is still taken exactly once. Only
  // the prefill-sized instantiations (cached new residual) carry the test: only their
  // plans loop, and in the decode kernels its few scalar instructions ahead of the first
  // loads cost 0.7% at P = 8, 80 x 4096.
  uint32_t block = blockIdx.x;
  if constexpr (CACHED_RESIDUAL) {
    const uint32_t blocks_per_xcd = gridDim.x / kXcds;
    if (rows_per_sweep < num_rows && gridDim.x % kXcds == 0u)
      block = (blockIdx.x % kXcds) * blocks_per_xcd + blockIdx.x / kXcds;
  }
  int parity = 0;
  for (uint32_t row0 = block * static_cast<uint32_t>(rows_per_block); row0 < num_rows;
       row0 += rows_per_sweep, parity ^= 1) {
    const uint32_t row = row0 + static_cast<uint32_t>(team);
    const bool active = row < num_rows;
    // A team past the last token gets empty descriptors: it reads zeros, writes nothing,
    // and still takes part in the workgroup's barriers.
    const int64_t off = active ? static_cast<int64_t>(row) * row_bytes : 0;
    const int nbytes = active ? row_bytes : 0;

    // ---- exact sum (binary64): partials in order, then the residual
    // The (P + 1) * NPACK pack loads of this lane form one sequence, pack-major: pack k's
    // partials 0..P-1 then its residual, then pack k + 1. A window of load_window loads
    // stays in flight (load i + window is issued right after load i is consumed), and
    // as soon as a pack's residual arrives the pack is finished: rounded, its new
    // residual stored, its squares and x * w taken, while later packs are still loading.
    // Pinning each accumulation step in place keeps the compiler from deferring the adds
    // and holding every loaded pack ((P + 1) * NPACK * 4 VGPRs).
    constexpr int kLoads = (P + 1) * NPACK;
    constexpr bool kWideSum = sizeof(typename Fmt::AccScalar) == 8;
    constexpr int kWinMax = load_window<NPACK, P, QUANT, kWideSum, RAGGED>();
    // RAGGED: the partial pack's narrow loads (one entry of four words per input) lead
    // the sequence: they share the window's registers, their round trip overlaps the
    // packs', and they are summed first (in the pack accumulators, which are free
    // then), so only the rounded partial pack (4 VGPRs) is carried through the loop
    constexpr bool kTailEarly = RAGGED && tail_early<NPACK, P, QUANT>();
    constexpr int kPre = kTailEarly ? P + 1 : 0;
    constexpr int kSeq = kPre + kLoads;
    constexpr int kWin = kSeq < kWinMax ? kSeq : kWinMax;
    __amdgpu_buffer_rsrc_t in_rsrc[P + 1];
#pragma unroll
    for (int p = 0; p < P; ++p) in_rsrc[p] = row_rsrc(a.partials[p], off, nbytes);
    // no residual input: an empty range reads zeros (adding +0 changes no value)
    in_rsrc[P] = row_rsrc(a.residual, off, a.residual != nullptr ? nbytes : 0);
    auto load_at = [&](int i) -> u32x4 {
      const int k = i / (P + 1);
      const int p = i - k * (P + 1);
      return __builtin_amdgcn_raw_buffer_load_b128(in_rsrc[p], voff[k], 0, kNonTemporal);
    };
    // new residual not wanted: an empty range drops the stores
    const __amdgpu_buffer_rsrc_t res_rsrc =
        row_rsrc(a.residual_out, off, a.residual_out != nullptr ? nbytes : 0);
    typename Fmt::Acc acc[4];  // the sum of each element of the current pack
    // x * w per element, kept in fp32 registers, computed while later loads are still
    // in flight, so that only the multiplication by r is left after the row reduction.
    // With the binary64 sum (fp16) deeper launches keep the rounded new residual
    // packed instead (4 VGPRs per pack rather than 8) and recompute x * w from it and
    // the packed gamma where it is needed (the same fp32 operations give the same
    // values), to stay within the register budget; so do the five-pack launches of rows
    // ending in a partial pack, whose partial pack needs registers of its own.
    constexpr bool kKeepXw =
        NPACK <= kKeepXwMaxPacks || (!kWideSum && !(RAGGED && NPACK == kMaxPacksPerLane));
    u32x4 xr[NPACK];
    float xw_kept[kKeepXw ? NPACK : 1][8];
    auto xw_compute = [&](int k, float* out) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 x = Fmt::unpack(xr[k][w]);
        const f32x2 gm = Fmt::unpack(g[k][w]);
        out[2 * w] = x.x * (wb + gm.x);
        out[2 * w + 1] = x.y * (wb + gm.y);
      }
    };
    // x * w of the partial last pack (RAGGED), gathered from its slot by selects rather
    // than a branch per slot; false (and zeros) in every other lane
    auto xw_of_tail = [&](float* out) -> bool {
      bool any = false;
      u32x4 xs = {0u, 0u, 0u, 0u};
      u32x4 gs = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.0f;
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        const bool t = voff[k] == kTailOff;
        any = any || t;
        if constexpr (kKeepXw) {
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] = t ? xw_kept[k][e] : out[e];
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            xs[w] = t ? xr[k][w] : xs[w];
            gs[w] = t ? g[k][w] : gs[w];
          }
        }
      }
      if constexpr (!kKeepXw) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x2 x = Fmt::unpack(xs[w]);
          const f32x2 gm = Fmt::unpack(gs[w]);
          out[2 * w] = x.x * (wb + gm.x);
          out[2 * w + 1] = x.y * (wb + gm.y);
        }
      }
      return any;
    };
    auto xw_of = [&](int k, float* out) {
      if constexpr (kKeepXw) {
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = xw_kept[k][e];
      } else {
        xw_compute(k, out);
      }
    };
    float ss = 0.0f;
    uint32_t m = 0u;  // max |x * w| as fp32 bits (NaN sorts above inf)
    uint32_t mpk[NPACK];  // the same per pack (per-group scales)
    u32x4 win[kWin];
    // The partial pack's owner loads it; every other lane's offsets fall outside the
    // row (zeros, no memory request), so the entries need no branch.
    bool tail_mine = false;
    if constexpr (RAGGED) {
#pragma unroll
      for (int k = 0; k < NPACK; ++k) tail_mine = tail_mine || voff[k] == kTailOff;
    }
    auto load_seq = [&](int j) -> u32x4 {
      if (j < kPre) return tail_load<kNonTemporal>(in_rsrc[j], tail_at_lane(H, 2, tail_mine));
      return load_at(j - kPre);
    };
    if constexpr (RAGGED) {
#pragma unroll
      for (int j = 0; j < kWin; ++j) win[j] = load_seq(j);
    } else {
#pragma unroll
      for (int i = 0; i < kWin; ++i) win[i] = load_at(i);
    }
    // gamma stays packed (4 VGPRs per pack): hide its loop invariance so the compiler
    // does not hoist the unpacked weights (8 VGPRs per pack) out of the loop. The pin
    // comes after the row's first loads are issued: it makes the wave wait for gamma,
    // and waiting before issuing them would put gamma's round trip ahead of the row's.
#pragma unroll
    for (int k = 0; k < NPACK; ++k) asm volatile("" : "+v"(g[k]));
    u32x4 xt = {0u, 0u, 0u, 0u};  // the partial pack's new residual (RAGGED)
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      // the partial pack's input j, summed in the same order as a whole pack's
      if (tail_wave) {
        u32x4 v = tail_merge(win[j % kWin], tail_at(H, 2).last_dw);
        if constexpr (kWideSum) asm volatile("" : "+v"(v));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const typename Fmt::Acc t = __builtin_convertvector(Fmt::unpack(v[w]), typename Fmt::Acc);
          if (j == 0) acc[w] = t;
          else acc[w] += t;
          asm volatile("" : "+v"(acc[w].x), "+v"(acc[w].y));
        }
        if (j == kPre - 1) {
#pragma unroll
          for (int w = 0; w < 4; ++w) xt[w] = Fmt::pack_sum(acc[w]);
        }
      }
      if (j + kWin < kSeq) win[j % kWin] = load_seq(j + kWin);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int j = i + kPre;  // position in the load sequence
      const int k = i / (P + 1);
      const int p = i - k * (P + 1);
      u32x4 v = win[j % kWin];
      // binary64 sum: widened only here, after the previous load's accumulation;
      // otherwise the compiler may widen later loads early, holding 16 more VGPRs per
      // load, which spills the deeper windows (the binary32 sum needs no such order,
      // which costs time where it is not needed)
      if constexpr (kWideSum) asm volatile("" : "+v"(v));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const typename Fmt::Acc t = __builtin_convertvector(Fmt::unpack(v[w]), typename Fmt::Acc);
        if (p == 0) acc[w] = t;
        else acc[w] += t;
        asm volatile("" : "+v"(acc[w].x), "+v"(acc[w].y));
      }
      if (i + kWin < kLoads) win[j % kWin] = load_at(i + kWin);
      if (p == P) {
        // pack k complete: round once to storage (the new residual), store it; squares
        // (and, when quantising, max |x * w|) of this lane (lanes past the row end hold
        // zeros)
        mpk[k] = 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          xr[k][w] = Fmt::pack_sum(acc[w]);
          const f32x2 x = Fmt::unpack(xr[k][w]);
          ss = fmaf(x.x, x.x, ss);
          ss = fmaf(x.y, x.y, ss);
          if constexpr (kKeepXw) {
            const f32x2 gm = Fmt::unpack(g[k][w]);
            float xw0 = x.x * (wb + gm.x);
            float xw1 = x.y * (wb + gm.y);
            // computed here, while later loads are in flight: left to itself the compiler
            // sinks these products below the row reduction, onto the row's critical path.
            // Pinned in the decode-sized launches (new residual streamed out), whose kernel
            // ends with that path (0.8% faster at P = 8, 80 x 4096 bf16); prefill-sized
            // launches hide it behind other rows' loads and keep the registers (pinned
            // there, P = 2, 2048 x 5120 was 0.2% slower), and deeper launches would spill
            // holding the products
            if constexpr (NPACK <= kPinXwMaxPacks && !CACHED_RESIDUAL)
              asm volatile("" : "+v"(xw0), "+v"(xw1));
            xw_kept[k][2 * w] = xw0;
            xw_kept[k][2 * w + 1] = xw1;
            if (QUANT != kQuantNone)
              mpk[k] = max(mpk[k], max(__float_as_uint(xw0) & 0x7fffffffu,
                                       __float_as_uint(xw1) & 0x7fffffffu));
          }
        }
        if (!kKeepXw && QUANT != kQuantNone) {
          float v[8];
          xw_compute(k, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) mpk[k] = max(mpk[k], __float_as_uint(v[e]) & 0x7fffffffu);
        }
        m = max(m, mpk[k]);
        __builtin_amdgcn_raw_buffer_store_b128(xr[k], res_rsrc, voff[k], 0,
                                               CACHED_RESIDUAL ? 0 : kNonTemporal);
      }
    }

    // ---- the partial last pack (RAGGED): summed in the same order as a whole pack
    // (above, or here at five packs per lane) and finished in its slot like the loop does
    if constexpr (RAGGED && !kTailEarly) {
      if (tail_wave) {
        bool mine = false;
#pragma unroll
        for (int k = 0; k < NPACK; ++k) mine = mine || voff[k] == kTailOff;
        u32x4 raw[P + 1];
#pragma unroll
        for (int p = 0; p <= P; ++p) raw[p] = tail_load<kNonTemporal>(in_rsrc[p], tail_at_lane(H, 2, mine));
#pragma unroll
        for (int p = 0; p <= P; ++p) {
          const u32x4 v = tail_merge(raw[p], tail_at(H, 2).last_dw);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const typename Fmt::Acc t = __builtin_convertvector(Fmt::unpack(v[w]), typename Fmt::Acc);
            if (p == 0) acc[w] = t;
            else acc[w] += t;
          }
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) xt[w] = Fmt::pack_sum(acc[w]);
      }
    }
    if constexpr (RAGGED) {
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        if (voff[k] != kTailOff) continue;
        mpk[k] = 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          xr[k][w] = xt[w];
          const f32x2 x = Fmt::unpack(xr[k][w]);
          ss = fmaf(x.x, x.x, ss);
          ss = fmaf(x.y, x.y, ss);
          if constexpr (kKeepXw) {
            const f32x2 gm = Fmt::unpack(g[k][w]);
            const float xw0 = x.x * (wb + gm.x);
            const float xw1 = x.y * (wb + gm.y);
            xw_kept[k][2 * w] = xw0;
            xw_kept[k][2 * w + 1] = xw1;
            if (QUANT != kQuantNone)
              mpk[k] = max(mpk[k], max(__float_as_uint(xw0) & 0x7fffffffu,
                                       __float_as_uint(xw1) & 0x7fffffffu));
          }
        }
        if (!kKeepXw && QUANT != kQuantNone) {
          float v[8];
          xw_compute(k, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) mpk[k] = max(mpk[k], __float_as_uint(v[e]) & 0x7fffffffu);
        }
        m = max(m, mpk[k]);
        tail_store<CACHED_RESIDUAL ? 0 : kNonTemporal>(xr[k], res_rsrc, tail_at(H, 2));
      }
    }

    // ---- row reductions: wave (DPP), then across the team's waves through LDS
    constexpr bool kRowMax = QUANT != kQuantNone && QUANT != kQuantDynamicGroup;
    float total = wave_sum(ss);
    if (kRowMax) m = wave_umax(m);
    if (waves_per_row > 1) {
      if ((tid & (kWave - 1)) == 0) {
        red_sum[parity][wave] = total;
        if (kRowMax) red_max[parity][wave] = m;
      }
      __syncthreads();
      const int w0 = team * waves_per_row;
      team_reduce<kRowMax>(red_sum[parity], red_max[parity], w0, waves_per_row, &total, &m);
    }
    // the dynamic codes' multiplier needs only the row max: computed here, beside r
    // (unconditionally, then selected, so that it interleaves with r's division)
    float mul_dynamic = 0.0f;
    if constexpr (QUANT == kQuantDynamic) {
      const float q = kE4m3Max / __uint_as_float(m);
      mul_dynamic = m != 0u ? q : 0.0f;
      asm volatile("" : "+v"(mul_dynamic));  // (left alone, the compiler sinks it to its use)
    }
    const float r = __builtin_amdgcn_rsqf(total / static_cast<float>(H) + a.eps);

    // ---- normalised output
    // (a row's partial last pack first: while every pack's values are still held, its
    // stores add no register pressure)
    if (QUANT == kQuantNone || a.norm_out != nullptr) {
      const __amdgpu_buffer_rsrc_t n_rsrc = row_rsrc(a.norm_out, off, nbytes);
      // r taken afresh inside the branch: x*w*r would otherwise be shared with the fp8
      // exact path and hoisted above the branch, onto the codes' critical path when
      // norm_out is not written (0.05 us at P = 4, 64 x 8192)
      float rn = r;
      if constexpr (QUANT != kQuantNone) asm volatile("" : "+v"(rn));
      if constexpr (RAGGED) {
        float v[8];
        if (xw_of_tail(v)) {
          u32x4 o;
#pragma unroll
          for (int w = 0; w < 4; ++w) o[w] = Fmt::pack(f32x2{v[2 * w] * rn, v[2 * w + 1] * rn});
          tail_store<kNonTemporal>(o, n_rsrc, tail_at(H, 2));
        }
      }
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        u32x4 o;
        float v[8];
        xw_of(k, v);
#pragma unroll
        for (int w = 0; w < 4; ++w) o[w] = Fmt::pack(f32x2{v[2 * w] * rn, v[2 * w + 1] * rn});
        __builtin_amdgcn_raw_buffer_store_b128(o, n_rsrc, voff[k], 0, kNonTemporal);
      }
    }

    // ---- fp8 epilogue
    if (QUANT == kQuantStatic || QUANT == kQuantDynamic) {
      float mul;    // fast path: code = E4M3(xw * mul)
      float denom;  // exact path: code = E4M3((xw * r) * (1 / denom))
      float amax = 0.0f;  // dynamic: the row's max |y|
      bool fast;
      if (QUANT == kQuantStatic) {
        const float S = static_scale;
        mul = r / S;
        denom = S;
        fast = finite_f32(r) && finite_f32(mul) && m < 0x7f800000u;
      } else {
        amax = amax_of(m, r);
        mul = mul_dynamic;  // r cancels from y / scale
        denom = amax;       // the exact path takes the scale of it
        // the scale (amax / 448, or 1 for a zero row) is finite exactly when amax is, so
        // the codes need not wait for that division; the scale is stored after them
        fast = finite_f32(r) && finite_f32(mul) && finite_f32(amax) && m < 0x7f800000u;
      }
      constexpr bool kDenomIsAmax = QUANT == kQuantDynamic;
      const __amdgpu_buffer_rsrc_t q_rsrc = row_rsrc(a.quant_out, off / 2, nbytes / 2);
      // fast holds for the whole row (r, mul and the row max are the team's). Taken
      // through a scalar register, it is one scalar branch around straight-line code for
      // all the row's packs, and marked likely, so that the fast path falls through and
      // the exact path's code (about 2 KB) is placed after the loop rather than between
      // the branch and the fast path, where the fast path jumped over it into instruction
      // cache lines not yet fetched.
      if (__builtin_expect(__builtin_amdgcn_readfirstlane(fast ? 1 : 0) != 0, 1)) {
        if constexpr (RAGGED) {
          float v[8];
          if (xw_of_tail(v)) tail_store_codes<kNonTemporal>(pack_codes_fast(v, mul), q_rsrc, tail_at(H, 1));
        }
#pragma unroll
        for (int k = 0; k < NPACK; ++k) {
          float v[8];
          xw_of(k, v);
          __builtin_amdgcn_raw_buffer_store_b64(pack_codes_fast(v, mul), q_rsrc, voff[k] / 2, 0,
                                                kNonTemporal);
        }
      } else {
        if constexpr (RAGGED) {
          float v[8];
          if (xw_of_tail(v))
            tail_store_codes<kNonTemporal>(pack_codes_exact<kDenomIsAmax>(v, r, denom), q_rsrc,
                                           tail_at(H, 1));
        }
#pragma unroll
        for (int k = 0; k < NPACK; ++k) {
          float v[8];
          xw_of(k, v);
          __builtin_amdgcn_raw_buffer_store_b64(pack_codes_exact<kDenomIsAmax>(v, r, denom), q_rsrc,
                                                voff[k] / 2, 0, kNonTemporal);
        }
      }
      if (QUANT == kQuantDynamic && active && lane == 0) {
        float am = amax;
        asm volatile("" : "+v"(am));  // after the codes, not ahead of them
        a.scale_out[row] = scale_of(am);
      }
    }
    if (QUANT == kQuantDynamicGroup) {
      // a 128-element group is 16 packs held by the 16 lanes of one DPP row (team
      // sizes are whole waves), so the group max needs no LDS
      const int64_t srow = active ? static_cast<int64_t>(row) * a.groups * 4 : 0;
      const __amdgpu_buffer_rsrc_t s_rsrc = row_rsrc(a.scale_out, srow, active ? a.groups * 4 : 0);
      const __amdgpu_buffer_rsrc_t q_rsrc = row_rsrc(a.quant_out, off / 2, nbytes / 2);
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        const uint32_t mg = row16_umax(mpk[k]);
        const float sc = scale_of(amax_of(mg, r));
        const float mul = (mg == 0u) ? 0.0f : kE4m3Max / __uint_as_float(mg);
        const bool fast = finite_f32(r) && finite_f32(mul) && finite_f32(sc) && mg < 0x7f800000u;
        float v[8];
        xw_of(k, v);
        if constexpr (RAGGED) {
          // the partial pack's group: pack H / 8, group H / 128, byte offset H / 32
          const bool tail = voff[k] == kTailOff;
          if ((lane & 15) == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), s_rsrc,
                                                  tail ? (H >> 5) & ~3 : voff[k] >> 6, 0, 0);
          const u32x2 q = pack_codes(v, mul, fast, r, sc);
          __builtin_amdgcn_raw_buffer_store_b64(q, q_rsrc, voff[k] / 2, 0, kNonTemporal);
          if (tail) tail_store_codes<kNonTemporal>(q, q_rsrc, tail_at(H, 1));
        } else {
          if ((lane & 15) == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), s_rsrc, voff[k] >> 6, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b64(pack_codes(v, mul, fast, r, sc), q_rsrc,
                                                voff[k] / 2, 0, kNonTemporal);
        }
      }
    }
    if (QUANT == kQuantDynamicTensor) {
      // codes wait for the tensor's max: record this row's max |y| and r
      if (active && lane == 0) {
        a.workspace[row] = amax_of(m, r);
        a.workspace[a.num_tokens + row] = r;
      }
    }
  }  // row loop
}

// ---------------------------------------------------------------- generic kernel
// Any H, any alignment: one workgroup per row (64..1024 lanes, chosen by the plan from
// H; a grid-stride loop over rows when the grid is capped), element loop. Pass 1 sums, rounds, writes residual_out (if wanted) and
// accumulates the sum of squares; pass 2 (dynamic only) takes the max |y|; pass 3
// writes norm_out / codes. Passes 2 and 3 re-read the elements this lane wrote, or
// recompute them when the new residual is not written (then no input was
// overwritten). Every element is read and written by one lane, so the in-place forms
// are safe here too. Each lane takes kGenUnroll elements per trip and issues all their
// loads before using any; a lane whose element of a trip lies past the row end loads
// its first element of that trip again (a valid address it owns) and discards it.
// Codes use the exact software conversion.
constexpr int kGenMaxThreads = 1024;
constexpr int kGenUnroll = 4;

// Sum of one element (partials in order, then the residual) in the format's accumulator
// type, returned as the binary32 value that rounds to the storage type like the sum (P
// fixed, or taken from the arguments when P is 0).
template <typename Fmt, int P = 0>
__device__ __forceinline__ float generic_sum(const KernelArgs& a, int64_t i) {
  typename Fmt::AccScalar s = Fmt::load1(a.partials[0], i);
  if (P > 0) {
#pragma unroll
    for (int p = 1; p < P; ++p) s += Fmt::load1(a.partials[p], i);
  } else {
#pragma unroll
    for (int p = 1; p < kMaxPartials; ++p)
      if (p < a.num_partials) s += Fmt::load1(a.partials[p], i);
  }
  if (a.residual != nullptr) s += Fmt::load1(a.residual, i);
  return Fmt::sum_to_f32(s);
}

template <typename Fmt, int P, int QUANT>
__global__ void __launch_bounds__(kGenMaxThreads)
far_generic_kernel(const KernelArgs a) {
  // reduction slots, double buffered by row-loop parity (as in the vector kernel)
  static_assert(kGenMaxThreads / kWave == kMaxWavesPerBlock, "the slot reduction covers 16 waves");
  __shared__ float red_sum[2][kGenMaxThreads / kWave];
  __shared__ uint32_t red_max[2][kGenMaxThreads / kWave];
  const int tid = static_cast<int>(threadIdx.x);
  const int nthr = static_cast<int>(blockDim.x);  // a multiple of 64
  const int nwaves = nthr / kWave;
  const int wave = tid / kWave;
  const int H = a.hidden;
  const int64_t trip = static_cast<int64_t>(nthr) * kGenUnroll;
  const float wb = a.weight_bias;
  int parity = 0;
  // one row per workgroup; with fewer workgroups than rows (very large T) each
  // workgroup loops over rows (the bound is uniform across the workgroup)
  for (int64_t row = blockIdx.x; row < a.num_tokens; row += gridDim.x, parity ^= 1) {
    const int64_t off = row * static_cast<int64_t>(H);
    auto x_at = [&](int64_t h) -> float {
      return a.residual_out != nullptr ? Fmt::load1(a.residual_out, off + h)
                                       : Fmt::round1(generic_sum<Fmt, P>(a, off + h));
    };

    float ss = 0.0f;
    for (int64_t h0 = tid; h0 < H; h0 += trip) {
      float x[kGenUnroll];
#pragma unroll
      for (int u = 0; u < kGenUnroll; ++u) {
        const int64_t h = h0 + static_cast<int64_t>(u) * nthr;
        x[u] = Fmt::round1(generic_sum<Fmt, P>(a, off + (h < H ? h : h0)));
      }
#pragma unroll
      for (int u = 0; u < kGenUnroll; ++u) {
        const int64_t h = h0 + static_cast<int64_t>(u) * nthr;
        if (h < H) {
          if (a.residual_out != nullptr) Fmt::store1(a.residual_out, off + h, x[u]);
          ss = fmaf(x[u], x[u], ss);
        }
      }
    }
    float total = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) red_sum[parity][wave] = total;
    __syncthreads();
    team_reduce<false>(red_sum[parity], nullptr, 0, nwaves, &total, nullptr);
    const float r = __builtin_amdgcn_rsqf(total / static_cast<float>(H) + a.eps);
    auto y_at = [&](int64_t h) -> float { return (x_at(h) * r) * (wb + Fmt::load1(a.gamma, h)); };
    // y of this lane's elements of one trip (clamped like pass 1)
    auto y_trip = [&](int64_t h0, float* y) {
#pragma unroll
      for (int u = 0; u < kGenUnroll; ++u) {
        const int64_t h = h0 + static_cast<int64_t>(u) * nthr;
        y[u] = y_at(h < H ? h : h0);
      }
    };

    if (QUANT == kQuantDynamicGroup) {
      // each lane takes whole groups: max over its group, then its codes
      constexpr int kG = 8;  // elements per step inside a group
      for (int64_t g = tid; g < a.groups; g += nthr) {
        const int64_t h0 = g * kFp8Group;
        const int64_t h1 = h0 + kFp8Group < H ? h0 + kFp8Group : H;
        uint32_t m = 0u;
        for (int64_t hb = h0; hb < h1; hb += kG) {
          float y[kG];
#pragma unroll
          for (int u = 0; u < kG; ++u) y[u] = y_at(hb + u < h1 ? hb + u : h0);
#pragma unroll
          for (int u = 0; u < kG; ++u)
            if (hb + u < h1) m = max(m, __float_as_uint(y[u]) & 0x7fffffffu);
        }
        const float sc = scale_of(__uint_as_float(m));
        a.scale_out[row * a.groups + g] = sc;
        const float inv = 1.0f / sc;
        for (int64_t hb = h0; hb < h1; hb += kG) {
          float y[kG];
#pragma unroll
          for (int u = 0; u < kG; ++u) y[u] = y_at(hb + u < h1 ? hb + u : h0);
#pragma unroll
          for (int u = 0; u < kG; ++u) {
            if (hb + u < h1) {
              if (a.norm_out != nullptr) Fmt::store1(a.norm_out, off + hb + u, y[u]);
              a.quant_out[off + hb + u] = static_cast<uint8_t>(e4m3_code(y[u] * inv));
            }
          }
        }
      }
      continue;
    }

    float inv = 1.0f;
    if (QUANT == kQuantStatic) inv = 1.0f / a.scale[0];
    if (QUANT == kQuantDynamic || QUANT == kQuantDynamicTensor) {
      uint32_t m = 0u;
      for (int64_t h0 = tid; h0 < H; h0 += trip) {
        float y[kGenUnroll];
        y_trip(h0, y);
#pragma unroll
        for (int u = 0; u < kGenUnroll; ++u)
          if (h0 + static_cast<int64_t>(u) * nthr < H) m = max(m, __float_as_uint(y[u]) & 0x7fffffffu);
      }
      m = wave_umax(m);
      if ((tid & (kWave - 1)) == 0) red_max[parity][wave] = m;
      __syncthreads();
      m = team_umax(red_max[parity], 0, nwaves);
      if (QUANT == kQuantDynamicTensor) {
        if (tid == 0) {
          a.workspace[row] = __uint_as_float(m);
          a.workspace[a.num_tokens + row] = r;
        }
      } else {
        const float sc = scale_of(__uint_as_float(m));
        if (tid == 0) a.scale_out[row] = sc;
        inv = 1.0f / sc;
      }
    }
    for (int64_t h0 = tid; h0 < H; h0 += trip) {
      float y[kGenUnroll];
      y_trip(h0, y);
#pragma unroll
      for (int u = 0; u < kGenUnroll; ++u) {
        const int64_t h = h0 + static_cast<int64_t>(u) * nthr;
        if (h < H) {
          if (a.norm_out != nullptr) Fmt::store1(a.norm_out, off + h, y[u]);
          if (QUANT == kQuantStatic || QUANT == kQuantDynamic)
            a.quant_out[off + h] = static_cast<uint8_t>(e4m3_code(y[u] * inv));
        }
      }
    }
  }  // row loop
}

// ---------------------------------------------------------------- per-tensor scale
// Second and third kernels of the per-tensor dynamic mode. The first (vector or
// generic kernel) left each row's max |y| in workspace[0, T) and its r in
// workspace[T, 2T). One workgroup reduces the maxima to the tensor scale; then an
// elementwise pass turns x * w * r / scale into codes, with x re-read from the new
// residual (or recomputed from the inputs when it was not written).
template <int kThreads>
__global__ void __launch_bounds__(kThreads)
far_tensor_scale_kernel(const float* __restrict__ row_max, int64_t T, float* __restrict__ scale_out) {
  __shared__ uint32_t red[kThreads / kWave];
  uint32_t m = 0u;
  for (int64_t t = threadIdx.x; t < T; t += kThreads) m = max(m, __float_as_uint(row_max[t]) & 0x7fffffffu);
  m = wave_umax(m);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
    for (int w = 0; w < kThreads / kWave; ++w) t = max(t, red[w]);
    scale_out[0] = scale_of(__uint_as_float(t));
  }
}

constexpr int kQuantThreads = 256;

// VEC: one 16-byte pack (8 elements) per lane and step, a row's partial last pack (H % 8
// elements) element by element; otherwise one element per lane and step. Grid-stride
// over the tensor.
template <typename Fmt, bool VEC>
__global__ void __launch_bounds__(kQuantThreads)
far_tensor_quant_kernel(const KernelArgs a) {
  const int H = a.hidden;
  const int units_per_row = VEC ? (H + 7) / 8 : H;
  const int64_t units = a.num_tokens * units_per_row;
  const float sc = a.scale_out[0];
  const float inv_sc = 1.0f / sc;
  const float wb = a.weight_bias;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x; i < units;
       i += static_cast<int64_t>(gridDim.x) * kQuantThreads) {
    const int64_t row = i / units_per_row;
    const int col = static_cast<int>(i - row * units_per_row);
    const float r = a.workspace[a.num_tokens + row];
    const float mul = r * inv_sc;
    if (VEC) {
      const int64_t e0 = row * H + col * 8;
      const int n = H - col * 8 < 8 ? H - col * 8 : 8;  // elements of this pack
      float x[8];
      float gm[8];
      if (n == 8) {
        u32x4 v;  // tensors need only element alignment: byte copies, one 16-byte load
        if (a.residual_out != nullptr) {
          __builtin_memcpy(&v, static_cast<const uint16_t*>(a.residual_out) + e0, sizeof(v));
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x2 t = Fmt::unpack(v[w]);
            x[2 * w] = t.x;
            x[2 * w + 1] = t.y;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = Fmt::round1(generic_sum<Fmt>(a, e0 + e));
        }
        __builtin_memcpy(&v, static_cast<const uint16_t*>(a.gamma) + col * 8, sizeof(v));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x2 t = Fmt::unpack(v[w]);
          gm[2 * w] = t.x;
          gm[2 * w + 1] = t.y;
        }
      } else {
        // the row's partial last pack: only its n elements are read (zeros beyond)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = 0.0f;
          gm[e] = 0.0f;
          if (e < n) {
            x[e] = a.residual_out != nullptr ? Fmt::load1(a.residual_out, e0 + e)
                                             : Fmt::round1(generic_sum<Fmt>(a, e0 + e));
            gm[e] = Fmt::load1(a.gamma, col * 8 + e);
          }
        }
      }
      float xw[8];
      uint32_t mk = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xw[e] = x[e] * (wb + gm[e]);
        mk = max(mk, __float_as_uint(xw[e]) & 0x7fffffffu);
      }
      const bool fast = finite_f32(mul) && finite_f32(r) && mk < 0x7f800000u;
      const u32x2 codes = pack_codes(xw, mul, fast, r, sc);
      if (n == 8) {
        __builtin_memcpy(a.quant_out + e0, &codes, sizeof(codes));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < n) a.quant_out[e0 + e] = static_cast<uint8_t>((e < 4 ? codes.x : codes.y) >> (8 * (e & 3)));
      }
    } else {
      const int64_t e = row * H + col;
      const float x = a.residual_out != nullptr ? Fmt::load1(a.residual_out, e)
                                                : Fmt::round1(generic_sum<Fmt>(a, e));
      const float y = (x * r) * (wb + Fmt::load1(a.gamma, col));
      a.quant_out[e] = static_cast<uint8_t>(e4m3_code(y * inv_sc));
    }
  }
}

}  // namespace far
