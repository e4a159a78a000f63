// far_kernels.hpp -- HIP kernels of the fused "sum of partials + residual add + RMSNorm
// (+ fp8 quant)" epilogue, written for gfx950 (CDNA4, wave64).
//
// The operation is defined on page "vllm.models.common.ops.fused_allreduce_rms_norm"
// (fused_allreduce_rms_norm: (normed_output, new_residual) = norm(all_reduce(partials),
// residual), fp32 accumulation, weight_bias + gamma) and page "vllm.compilation.fusion"
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
// up to 2% over 10.
template <int NPACK, int P, int QUANT>
constexpr int load_window() {
  return QUANT == kQuantDynamicGroup
             ? (NPACK <= 2 ? 12 : (NPACK == 3 ? 8 : 5))
             : (NPACK <= 2 ? 16
                : NPACK == 3 ? (P >= 5 ? 21 : 10)
                : NPACK == 4 ? (P >= 2 && P <= 4 ? 16 : 5)
                             : (P <= 4 ? 9 : 6));
}

// Packs per lane a mode supports: the per-group epilogue needs a little more than the
// others, and at five packs it would spill.
constexpr int max_packs_for(int quant) { return quant == kQuantDynamicGroup ? 4 : kMaxPacksPerLane; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// ---------------------------------------------------------------- storage formats
// Two storage values per 32-bit word; conversions to storage round to nearest even
// (gfx950 has a packed bf16 convert; fp16 converts honour the default RNE mode).
struct Bf16 {
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
};

struct Fp16 {
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
};

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

// Eight codes of one pack: hardware conversion when `fast` (every value finite and
// the multiplier finite), else the exact software conversion of (xw * r) * inv_y.
__device__ __forceinline__ u32x2 pack_codes(const float* xw, float mul, bool fast, float r,
                                            float inv_y) {
  u32x2 q;
  if (fast) {
    q.x = e4m3_pair_fast(xw[0] * mul, xw[1] * mul) | (e4m3_pair_fast(xw[2] * mul, xw[3] * mul) << 16);
    q.y = e4m3_pair_fast(xw[4] * mul, xw[5] * mul) | (e4m3_pair_fast(xw[6] * mul, xw[7] * mul) << 16);
  } else {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (xw[e] * r) * inv_y;
    q.x = e4m3_pack4(y[0], y[1], y[2], y[3]);
    q.y = e4m3_pack4(y[4], y[5], y[6], y[7]);
  }
  return q;
}

// Buffer resource (V#) over `bytes` bytes at `base`: raw addressing (stride 0), so a
// load at a byte offset >= bytes returns zeros and a store there is dropped by the
// hardware range check. Rows are multiples of 16 bytes and offsets are pack-aligned,
// so a 16-byte pack is either wholly inside or wholly outside.
constexpr int kRsrcWord3 = 0x00020000;  // GFX9 family: 32-bit data format, raw buffer
constexpr int kNonTemporal = 2;         // cache-policy bit: streamed once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t byte_off,
                                                           int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(base)) + byte_off, 0, bytes, kRsrcWord3);
}

template <typename Fmt, int P, int NPACK, int QUANT>
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
  int voff[NPACK];  // byte offset of each of this lane's packs inside a row (may be
                    // past the end: then loads read zeros and stores are dropped)
#pragma unroll
  for (int k = 0; k < NPACK; ++k) voff[k] = (lane + k * team_lanes) * 16;

  // ---- gamma: shared by every row, loaded once per team and kept in registers
  const __amdgpu_buffer_rsrc_t g_rsrc = row_rsrc(a.gamma, 0, row_bytes);
  u32x4 g[NPACK];
#pragma unroll
  for (int k = 0; k < NPACK; ++k) g[k] = __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, voff[k], 0, 0);
  const float wb = a.weight_bias;

  // Grid-stride loop over rows: with fewer workgroups than row groups, a team starts
  // the loads of its next row right after the stores of the current one, so reads and
  // writes of different rows overlap. The loop bound is uniform across the workgroup
  // (every team takes the same number of trips, as the barriers require).
  const int64_t rows_per_sweep = static_cast<int64_t>(gridDim.x) * rows_per_block;
  int parity = 0;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * rows_per_block; row0 < a.num_tokens;
       row0 += rows_per_sweep, parity ^= 1) {
    const int64_t row = row0 + team;
    const bool active = row < a.num_tokens;
    // A team past the last token gets empty descriptors: it reads zeros, writes nothing,
    // and still takes part in the workgroup's barriers.
    const int64_t off = active ? row * static_cast<int64_t>(row_bytes) : 0;
    const int nbytes = active ? row_bytes : 0;

    // ---- sum in fp32: partials in order, then the residual
    // The (P + 1) * NPACK pack loads of this lane form one sequence, pack-major: pack k's
    // partials 0..P-1 then its residual, then pack k + 1. A window of load_window loads
    // stays in flight (load i + window is issued right after load i is consumed), and
    // as soon as a pack's residual arrives the pack is finished: rounded, its new
    // residual stored, its squares and x * w taken, while later packs are still loading.
    // Pinning each accumulation step in place keeps the compiler from deferring the adds
    // and holding every loaded pack ((P + 1) * NPACK * 4 VGPRs).
    constexpr int kLoads = (P + 1) * NPACK;
    constexpr int kWin = kLoads < load_window<NPACK, P, QUANT>() ? kLoads : load_window<NPACK, P, QUANT>();
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
    f32x2 acc[4];
    // x * w per element, kept as fp32 registers (8 per pack)
    float xw[NPACK][8];
    auto xw_of = [&](int k, float* out) {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = xw[k][e];
    };
    float ss = 0.0f;
    uint32_t m = 0u;  // max |x * w| as fp32 bits (NaN sorts above inf)
    uint32_t mpk[NPACK];  // the same per pack (per-group scales)
    u32x4 win[kWin];
#pragma unroll
    for (int i = 0; i < kWin; ++i) win[i] = load_at(i);
    // gamma stays packed (4 VGPRs per pack): hide its loop invariance so the compiler
    // does not hoist the unpacked weights (8 VGPRs per pack) out of the loop. The pin
    // comes after the row's first loads are issued: it makes the wave wait for gamma,
    // and waiting before issuing them would put gamma's round trip ahead of the row's.
#pragma unroll
    for (int k = 0; k < NPACK; ++k) asm volatile("" : "+v"(g[k]));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int k = i / (P + 1);
      const int p = i - k * (P + 1);
      const u32x4 v = win[i % kWin];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (p == 0) acc[w] = Fmt::unpack(v[w]);
        else acc[w] += Fmt::unpack(v[w]);
        asm volatile("" : "+v"(acc[w].x), "+v"(acc[w].y));
      }
      if (i + kWin < kLoads) win[i % kWin] = load_at(i + kWin);
      if (p == P) {
        // pack k complete: round once to storage (the new residual), store it; squares
        // and x * w of this lane (lanes past the row end hold zeros)
        u32x4 xr;
        mpk[k] = 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          xr[w] = Fmt::pack(acc[w]);
          const f32x2 x = Fmt::unpack(xr[w]);
          const f32x2 gm = Fmt::unpack(g[k][w]);
          ss = fmaf(x.x, x.x, ss);
          ss = fmaf(x.y, x.y, ss);
          const float xw0 = x.x * (wb + gm.x);
          const float xw1 = x.y * (wb + gm.y);
          xw[k][2 * w] = xw0;
          xw[k][2 * w + 1] = xw1;
          if (QUANT != kQuantNone) {
            const uint32_t a0 = __float_as_uint(xw0) & 0x7fffffffu;
            const uint32_t a1 = __float_as_uint(xw1) & 0x7fffffffu;
            mpk[k] = max(mpk[k], max(a0, a1));
          }
        }
        m = max(m, mpk[k]);
        __builtin_amdgcn_raw_buffer_store_b128(xr, res_rsrc, voff[k], 0, kNonTemporal);
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
      total = 0.0f;
      const int w0 = team * waves_per_row;
      for (int w = 0; w < waves_per_row; ++w) total += red_sum[parity][w0 + w];
      if (kRowMax) {
        m = 0u;
        for (int w = 0; w < waves_per_row; ++w) m = max(m, red_max[parity][w0 + w]);
      }
    }
    const float r = __builtin_amdgcn_rsqf(total / static_cast<float>(H) + a.eps);

    // ---- normalised output
    if (QUANT == kQuantNone || a.norm_out != nullptr) {
      const __amdgpu_buffer_rsrc_t n_rsrc = row_rsrc(a.norm_out, off, nbytes);
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        u32x4 o;
        float v[8];
        xw_of(k, v);
#pragma unroll
        for (int w = 0; w < 4; ++w) o[w] = Fmt::pack(f32x2{v[2 * w] * r, v[2 * w + 1] * r});
        __builtin_amdgcn_raw_buffer_store_b128(o, n_rsrc, voff[k], 0, kNonTemporal);
      }
    }

    // ---- fp8 epilogue
    if (QUANT == kQuantStatic || QUANT == kQuantDynamic) {
      float mul;    // fast path: code = E4M3(xw * mul)
      float inv_y;  // exact path: code = E4M3((xw * r) * inv_y)
      bool fast;
      if (QUANT == kQuantStatic) {
        const float S = a.scale[0];
        mul = r / S;
        inv_y = 1.0f / S;
        fast = finite_f32(r) && finite_f32(mul) && m < 0x7f800000u;
      } else {
        const float sc = scale_of(amax_of(m, r));
        if (active && lane == 0) a.scale_out[row] = sc;
        mul = (m == 0u) ? 0.0f : kE4m3Max / __uint_as_float(m);  // r cancels from y / scale
        inv_y = 1.0f / sc;
        fast = finite_f32(r) && finite_f32(mul) && finite_f32(sc) && m < 0x7f800000u;
      }
      const __amdgpu_buffer_rsrc_t q_rsrc = row_rsrc(a.quant_out, off / 2, nbytes / 2);
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        float v[8];
        xw_of(k, v);
        __builtin_amdgcn_raw_buffer_store_b64(pack_codes(v, mul, fast, r, inv_y), q_rsrc,
                                              voff[k] / 2, 0, kNonTemporal);
      }
    }
    if (QUANT == kQuantDynamicGroup) {
      // a 128-element group is 16 packs held by the 16 lanes of one DPP row (team
      // sizes are whole waves), so the group max needs no LDS
      const int64_t srow = active ? row * static_cast<int64_t>(a.groups) * 4 : 0;
      const __amdgpu_buffer_rsrc_t s_rsrc = row_rsrc(a.scale_out, srow, active ? a.groups * 4 : 0);
      const __amdgpu_buffer_rsrc_t q_rsrc = row_rsrc(a.quant_out, off / 2, nbytes / 2);
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        const uint32_t mg = row16_umax(mpk[k]);
        const float sc = scale_of(amax_of(mg, r));
        const float mul = (mg == 0u) ? 0.0f : kE4m3Max / __uint_as_float(mg);
        const bool fast = finite_f32(r) && finite_f32(mul) && finite_f32(sc) && mg < 0x7f800000u;
        if ((lane & 15) == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), s_rsrc, voff[k] >> 6, 0, 0);
        float v[8];
        xw_of(k, v);
        __builtin_amdgcn_raw_buffer_store_b64(pack_codes(v, mul, fast, r, 1.0f / sc), q_rsrc,
                                              voff[k] / 2, 0, kNonTemporal);
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
// H), element loop. Pass 1 sums, rounds, writes residual_out (if wanted) and
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

// Sum of one element: partials in order, then the residual (P fixed, or taken from
// the arguments when P is 0).
template <typename Fmt, int P = 0>
__device__ __forceinline__ float generic_sum(const KernelArgs& a, int64_t i) {
  float s = Fmt::load1(a.partials[0], i);
  if (P > 0) {
#pragma unroll
    for (int p = 1; p < P; ++p) s += Fmt::load1(a.partials[p], i);
  } else {
#pragma unroll
    for (int p = 1; p < kMaxPartials; ++p)
      if (p < a.num_partials) s += Fmt::load1(a.partials[p], i);
  }
  if (a.residual != nullptr) s += Fmt::load1(a.residual, i);
  return s;
}

template <typename Fmt, int P, int QUANT>
__global__ void __launch_bounds__(kGenMaxThreads)
far_generic_kernel(const KernelArgs a) {
  __shared__ float red_sum[kGenMaxThreads / kWave];
  __shared__ uint32_t red_max[kGenMaxThreads / kWave];
  const int tid = static_cast<int>(threadIdx.x);
  const int nthr = static_cast<int>(blockDim.x);  // a multiple of 64
  const int nwaves = nthr / kWave;
  const int wave = tid / kWave;
  const int64_t row = blockIdx.x;
  const int H = a.hidden;
  const int64_t off = row * static_cast<int64_t>(H);
  const int64_t trip = static_cast<int64_t>(nthr) * kGenUnroll;
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
  if ((tid & (kWave - 1)) == 0) red_sum[wave] = total;
  __syncthreads();
  total = 0.0f;
  for (int w = 0; w < nwaves; ++w) total += red_sum[w];
  const float r = __builtin_amdgcn_rsqf(total / static_cast<float>(H) + a.eps);
  const float wb = a.weight_bias;
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
    return;
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
    if ((tid & (kWave - 1)) == 0) red_max[wave] = m;
    __syncthreads();
    m = 0u;
    for (int w = 0; w < nwaves; ++w) m = max(m, red_max[w]);
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

// VEC: one 16-byte pack (8 elements) per lane and step (H % 8 == 0, aligned tensors);
// otherwise one element per lane and step. Grid-stride over the tensor.
template <typename Fmt, bool VEC>
__global__ void __launch_bounds__(kQuantThreads)
far_tensor_quant_kernel(const KernelArgs a) {
  const int H = a.hidden;
  const int units_per_row = VEC ? H / 8 : H;
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
      float x[8];
      if (a.residual_out != nullptr) {
        u32x4 v;  // tensors need only element alignment: byte copies, one 16-byte load
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
      u32x4 gv;
      __builtin_memcpy(&gv, static_cast<const uint16_t*>(a.gamma) + col * 8, sizeof(gv));
      float xw[8];
      uint32_t mk = 0u;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 gm = Fmt::unpack(gv[w]);
        xw[2 * w] = x[2 * w] * (wb + gm.x);
        xw[2 * w + 1] = x[2 * w + 1] * (wb + gm.y);
        mk = max(mk, max(__float_as_uint(xw[2 * w]) & 0x7fffffffu, __float_as_uint(xw[2 * w + 1]) & 0x7fffffffu));
      }
      const bool fast = finite_f32(mul) && finite_f32(r) && mk < 0x7f800000u;
      const u32x2 codes = pack_codes(xw, mul, fast, r, inv_sc);
      __builtin_memcpy(a.quant_out + e0, &codes, sizeof(codes));
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
