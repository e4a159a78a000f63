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
// that make each wave instruction read 1 KiB of contiguous row, all of a lane's loads
// issued before they are consumed, the new residual row kept in registers (no second
// pass through memory), and one wave or LDS reduction per row. No MFMA: this is not a
// contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace far {

constexpr int kMaxPartials = 8;
constexpr int kWave = 64;
constexpr int kMaxWavesPerBlock = 16;
constexpr int kMaxPacksPerLane = 7;
// 16-byte loads each lane keeps in flight while summing: deeper for short rows, where
// the accumulators are few; with more packs per lane the accumulators take the
// registers and occupancy supplies the memory parallelism instead. Both keep every
// instantiation within 128 VGPRs without spilling.
template <int NPACK>
constexpr int load_window() { return NPACK <= 3 ? 8 : 4; }
constexpr float kE4m3Max = 448.0f;

enum Quant : int { kQuantNone = 0, kQuantStatic = 1, kQuantDynamic = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Everything a launch needs, passed by value in the kernel arguments (the partial
// pointers included, so no device-side pointer table is needed).
struct KernelArgs {
  const void* partials[kMaxPartials];
  const void* residual;
  const void* gamma;
  void* residual_out;
  void* norm_out;       // may be null with quantisation
  uint8_t* quant_out;   // fp8 e4m3fn codes
  float* scale_out;     // [T] per-token scales (dynamic)
  const float* scale;   // [1] static scale
  int64_t num_tokens;
  int32_t hidden;
  int32_t num_partials;
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
// (8 storage elements each), and is the only lane that reads or writes those
// elements, so residual_out may alias residual or partials[0]: every element is read
// before the same lane writes it.
// Workgroups of up to 1024 lanes: the compiler then keeps each wave within 128 VGPRs,
// four waves per SIMD, which still leaves tens of KiB of loads in flight per CU.
constexpr int kVecMaxThreads = 1024;

template <typename Fmt, int P, int NPACK, int QUANT>
__global__ void __launch_bounds__(kVecMaxThreads)
far_vec_kernel(const KernelArgs a, const int waves_per_row, const int rows_per_block) {
  __shared__ float red_sum[kMaxWavesPerBlock];
  __shared__ uint32_t red_max[kMaxWavesPerBlock];

  const int team_lanes = waves_per_row * kWave;
  const int tid = static_cast<int>(threadIdx.x);
  // A team is a whole number of waves, so the team (and the row) is uniform across a
  // wave: compute them as scalars so that every row address is a scalar base plus a
  // 32-bit per-lane byte offset (the global_load saddr form).
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave / waves_per_row;
  const int lane = tid - team * team_lanes;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * rows_per_block + team;
  const bool active = row < a.num_tokens;
  const int H = a.hidden;
  const int packs = H >> 3;
  // Loads are never predicated: a lane past the end of its row re-reads the row's last
  // pack and a team past the last token re-reads the last row, so every load stays in
  // bounds and the whole load/accumulate phase is one basic block the compiler can
  // schedule freely. Only the stores are predicated.
  const int64_t load_row = active ? row : a.num_tokens - 1;
  const int64_t row_off = load_row * static_cast<int64_t>(H);  // elements, uniform
  uint32_t boff[NPACK];  // byte offset of each of this lane's packs inside the row
#pragma unroll
  for (int k = 0; k < NPACK; ++k) boff[k] = static_cast<uint32_t>(min(lane + k * team_lanes, packs - 1)) * 16u;
  auto row_pack = [&](const void* base, int k) -> const u32x4* {
    return reinterpret_cast<const u32x4*>(
        reinterpret_cast<const char*>(static_cast<const uint16_t*>(base) + row_off) + boff[k]);
  };

  // ---- sum in fp32: partials in order, then the residual
  // The (P + 1) * NPACK pack loads of this lane form one sequence, tensor-major, so
  // each accumulator receives partial 0, 1, ..., P-1, then the residual. A window of
  // load_window loads is kept in flight: load i + window is issued right after load i
  // is consumed. Pinning each accumulation step in place keeps the compiler from
  // deferring the adds and holding every loaded pack ((P + 1) * NPACK * 4 registers).
  constexpr int kLoads = (P + 1) * NPACK;
  constexpr int kWin = kLoads < load_window<NPACK>() ? kLoads : load_window<NPACK>();
  auto load_at = [&](int i) -> u32x4 {
    const int p = i / NPACK;
    const int k = i - p * NPACK;
    const void* base = p < P ? a.partials[p < P ? p : 0] : a.residual;
    return __builtin_nontemporal_load(row_pack(base, k));
  };
  f32x2 acc[NPACK][4];
  u32x4 win[kWin];
#pragma unroll
  for (int i = 0; i < kWin; ++i) win[i] = load_at(i);
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = i / NPACK;
    const int k = i - p * NPACK;
    const u32x4 v = win[i % kWin];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (p == 0) acc[k][w] = Fmt::unpack(v[w]);
      else acc[k][w] += Fmt::unpack(v[w]);
      // pin the accumulation here: without it the adds drift to the end of the block
      // and every loaded pack stays live until then
      asm volatile("" : "+v"(acc[k][w].x), "+v"(acc[k][w].y));
    }
    if (i + kWin < kLoads) win[i % kWin] = load_at(i + kWin);
  }

  // ---- round once to storage (the new residual), keep it in registers, store it
  uint32_t xr[NPACK][4];
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < NPACK; ++k) {
    float part = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      xr[k][w] = Fmt::pack(acc[k][w]);
      const f32x2 x = Fmt::unpack(xr[k][w]);
      part = fmaf(x.x, x.x, part);
      part = fmaf(x.y, x.y, part);
    }
    // a lane past the end of the row holds a copy of the last pack: it adds nothing
    ss += (lane + k * team_lanes < packs) ? part : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < NPACK; ++k) {
    const int j = lane + k * team_lanes;
    if (active && j < packs) {
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.residual_out) + row_off) + j;
      __builtin_nontemporal_store(u32x4{xr[k][0], xr[k][1], xr[k][2], xr[k][3]}, dst);
    }
  }

  // ---- row mean square: wave sum, then across the team's waves through LDS
  float total = wave_sum(ss);
  if (waves_per_row > 1) {
    if ((tid & (kWave - 1)) == 0) red_sum[wave] = total;
    __syncthreads();
    total = 0.0f;
    const int w0 = team * waves_per_row;
    for (int w = 0; w < waves_per_row; ++w) total += red_sum[w0 + w];
  }
  const float r = __builtin_amdgcn_rsqf(total / static_cast<float>(H) + a.eps);

  // ---- weight: gamma packs (shared by every row, so they stay in cache)
  u32x4 g[NPACK];
#pragma unroll
  for (int k = 0; k < NPACK; ++k) {
    g[k] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.gamma) + boff[k]);
  }
  const float wb = a.weight_bias;

  // y = x * r * (weight_bias + gamma), recomputed from registers where needed
  auto y_pair = [&](int k, int w) -> f32x2 {
    const f32x2 x = Fmt::unpack(xr[k][w]);
    const f32x2 gm = Fmt::unpack(g[k][w]);
    f32x2 y;
    y.x = (x.x * r) * (wb + gm.x);
    y.y = (x.y * r) * (wb + gm.y);
    return y;
  };

  if (QUANT == kQuantNone || a.norm_out != nullptr) {
#pragma unroll
    for (int k = 0; k < NPACK; ++k) {
      const int j = lane + k * team_lanes;
      if (active && j < packs) {
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) o[w] = Fmt::pack(y_pair(k, w));
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.norm_out) + row_off) + j;
        __builtin_nontemporal_store(o, dst);
      }
    }
  }

  if (QUANT != kQuantNone) {
    float inv;
    if (QUANT == kQuantStatic) {
      inv = 1.0f / a.scale[0];
    } else {
      uint32_t m = 0u;
#pragma unroll
      for (int k = 0; k < NPACK; ++k) {
        uint32_t mk = 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x2 y = y_pair(k, w);
          const uint32_t ax = __float_as_uint(y.x) & 0x7fffffffu;
          const uint32_t ay = __float_as_uint(y.y) & 0x7fffffffu;
          mk = mk > ax ? mk : ax;
          mk = mk > ay ? mk : ay;
        }
        // a lane past the end of the row may have read a pack its owner has already
        // overwritten in place: it takes no part in the max
        mk = (lane + k * team_lanes < packs) ? mk : 0u;
        m = m > mk ? m : mk;
      }
      m = wave_umax(m);
      if (waves_per_row > 1) {
        if ((tid & (kWave - 1)) == 0) red_max[wave] = m;
        __syncthreads();
        m = 0u;
        const int w0 = team * waves_per_row;
        for (int w = 0; w < waves_per_row; ++w) m = m > red_max[w0 + w] ? m : red_max[w0 + w];
      }
      const float amax = __uint_as_float(m);
      const float sc = (m == 0u) ? 1.0f : amax / kE4m3Max;
      if (active && lane == 0) a.scale_out[row] = sc;
      inv = 1.0f / sc;
    }
#pragma unroll
    for (int k = 0; k < NPACK; ++k) {
      const int j = lane + k * team_lanes;
      if (active && j < packs) {
        const f32x2 y0 = y_pair(k, 0), y1 = y_pair(k, 1), y2 = y_pair(k, 2), y3 = y_pair(k, 3);
        u32x2 q;
        q.x = e4m3_pack4(y0.x * inv, y0.y * inv, y1.x * inv, y1.y * inv);
        q.y = e4m3_pack4(y2.x * inv, y2.y * inv, y3.x * inv, y3.y * inv);
        u32x2* dst = reinterpret_cast<u32x2*>(a.quant_out + row_off) + j;
        __builtin_nontemporal_store(q, dst);
      }
    }
  }
}

// ---------------------------------------------------------------- generic kernel
// Any H, any alignment: one workgroup of GEN_THREADS lanes per row, element loop.
// Pass 1 sums, rounds and writes residual_out and accumulates the sum of squares;
// pass 2 (dynamic only) re-reads the row this lane wrote and takes the max |y|;
// pass 3 writes norm_out / codes. Every element is read and written by one lane, so
// the in-place forms are safe here too.
constexpr int kGenThreads = 256;

template <typename Fmt, int QUANT>
__global__ void __launch_bounds__(kGenThreads)
far_generic_kernel(const KernelArgs a) {
  __shared__ float red_sum[kGenThreads / kWave];
  __shared__ uint32_t red_max[kGenThreads / kWave];
  const int tid = static_cast<int>(threadIdx.x);
  const int wave = tid / kWave;
  const int64_t row = blockIdx.x;
  const int H = a.hidden;
  const int64_t off = row * static_cast<int64_t>(H);

  float ss = 0.0f;
  for (int h = tid; h < H; h += kGenThreads) {
    float s = Fmt::load1(a.partials[0], off + h);
#pragma unroll
    for (int p = 1; p < kMaxPartials; ++p)
      if (p < a.num_partials) s += Fmt::load1(a.partials[p], off + h);
    s += Fmt::load1(a.residual, off + h);
    const float x = Fmt::round1(s);
    Fmt::store1(a.residual_out, off + h, x);
    ss = fmaf(x, x, ss);
  }
  float total = wave_sum(ss);
  if ((tid & (kWave - 1)) == 0) red_sum[wave] = total;
  __syncthreads();
  total = 0.0f;
  for (int w = 0; w < kGenThreads / kWave; ++w) total += red_sum[w];
  const float r = __builtin_amdgcn_rsqf(total / static_cast<float>(H) + a.eps);
  const float wb = a.weight_bias;

  float inv = 1.0f;
  if (QUANT == kQuantStatic) inv = 1.0f / a.scale[0];
  if (QUANT == kQuantDynamic) {
    uint32_t m = 0u;
    for (int h = tid; h < H; h += kGenThreads) {
      const float y = (Fmt::load1(a.residual_out, off + h) * r) * (wb + Fmt::load1(a.gamma, h));
      const uint32_t ay = __float_as_uint(y) & 0x7fffffffu;
      m = m > ay ? m : ay;
    }
    m = wave_umax(m);
    if ((tid & (kWave - 1)) == 0) red_max[wave] = m;
    __syncthreads();
    m = 0u;
    for (int w = 0; w < kGenThreads / kWave; ++w) m = m > red_max[w] ? m : red_max[w];
    const float sc = (m == 0u) ? 1.0f : __uint_as_float(m) / kE4m3Max;
    if (tid == 0) a.scale_out[row] = sc;
    inv = 1.0f / sc;
  }
  for (int h = tid; h < H; h += kGenThreads) {
    const float y = (Fmt::load1(a.residual_out, off + h) * r) * (wb + Fmt::load1(a.gamma, h));
    if (a.norm_out != nullptr) Fmt::store1(a.norm_out, off + h, y);
    if (QUANT != kQuantNone) a.quant_out[off + h] = static_cast<uint8_t>(e4m3_code(y * inv));
  }
}

}  // namespace far
