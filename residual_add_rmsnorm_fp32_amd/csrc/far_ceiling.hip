// far_ceiling.hip -- measurement aids for the benchmark (include/far_ceiling.h): streams
// that move the fused epilogue's bytes without its arithmetic, an empty kernel and a
// bounded sleep kernel. Written for gfx950 (wave64); independent of the epilogue's
// kernels.
#include <hip/hip_runtime.h>

#include <array>
#include <cstdint>
#include <utility>

#include "far_ceiling.h"

namespace {

constexpr int kWave = 64;
constexpr int kMaxIn = FAR_CEILING_MAX_INPUTS;
constexpr int kMaxPacks = 5;        // packs (or unrolled steps) per lane
constexpr int kMaxLoads = 24;       // inputs x packs per lane: loads in flight per lane
constexpr int kMaxThreads = 1024;
constexpr int64_t kMaxGrid = int64_t{1} << 20;
constexpr int kNonTemporal = 2;         // cache-policy bit: streamed once
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct StreamArgs {
  const void* in[kMaxIn];
  void* out_full;
  void* out2;
  float* out_row;
  int64_t count;      // rows (row kernel) or 16-byte packs per array (flat kernel)
  int32_t row_bytes;  // row kernel
  int32_t out2_half;
  int32_t waves_per_row;
  int32_t rows_per_block;
};

// Buffer resource over [base + off, base + off + bytes): loads past the end read zeros
// and stores there are dropped by the hardware's range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t off, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + off, 0,
                                           static_cast<int>(bytes), kRsrcWord3);
}

// Stores of one pack x (the XOR of the inputs' packs) to out_full and out2.
__device__ __forceinline__ void store_pack(u32x4 x, __amdgpu_buffer_rsrc_t o1, __amdgpu_buffer_rsrc_t o2,
                                           bool half, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(x, o1, voff, 0, kNonTemporal);
  if (half) {
    const u32x2 h = {x.x ^ x.z, x.y ^ x.w};
    __builtin_amdgcn_raw_buffer_store_b64(h, o2, voff / 2, 0, kNonTemporal);
  } else {
    const u32x4 r = {x.y, x.z, x.w, x.x};
    __builtin_amdgcn_raw_buffer_store_b128(r, o2, voff, 0, kNonTemporal);
  }
}

// Row-shaped stream: the fused kernel's launch shape (a team of waves per row, lane l
// holding packs l + k * team_lanes, teams per workgroup, grid-stride over rows) with
// every load of a row issued before any store.
template <int NIN, int NPACK>
__global__ void __launch_bounds__(kMaxThreads) far_ceiling_rows_kernel(const StreamArgs a) {
  const int team_lanes = a.waves_per_row * kWave;
  const int tid = static_cast<int>(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave / a.waves_per_row;
  const int lane = tid - team * team_lanes;
  const int rb = a.row_bytes;
  uint32_t voff[NPACK];
#pragma unroll
  for (int k = 0; k < NPACK; ++k) voff[k] = static_cast<uint32_t>(lane + k * team_lanes) * 16u;
  const bool half = a.out2_half != 0;
  const int64_t sweep = static_cast<int64_t>(gridDim.x) * a.rows_per_block;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * a.rows_per_block; row0 < a.count; row0 += sweep) {
    const int64_t row = row0 + team;
    const bool active = row < a.count;
    const int64_t off = active ? row * rb : 0;
    const uint32_t nb = active ? static_cast<uint32_t>(rb) : 0u;
    u32x4 v[NIN][NPACK];
#pragma unroll
    for (int i = 0; i < NIN; ++i) {
      const __amdgpu_buffer_rsrc_t r = rsrc(a.in[i], off, nb);
#pragma unroll
      for (int k = 0; k < NPACK; ++k) v[i][k] = __builtin_amdgcn_raw_buffer_load_b128(r, voff[k], 0, kNonTemporal);
    }
    const __amdgpu_buffer_rsrc_t o1 = rsrc(a.out_full, off, nb);
    const __amdgpu_buffer_rsrc_t o2 = rsrc(a.out2 != nullptr ? a.out2 : a.out_full, half ? off / 2 : off,
                                           a.out2 != nullptr ? (half ? nb / 2 : nb) : 0u);
    u32x4 first = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < NPACK; ++k) {
      u32x4 x = v[0][k];
#pragma unroll
      for (int i = 1; i < NIN; ++i) x ^= v[i][k];
      if (k == 0) first = x;
      store_pack(x, o1, o2, half, voff[k]);
    }
    if (a.out_row != nullptr && active && lane == 0) a.out_row[row] = __uint_as_float(first.x & 0x3fffffffu);
  }
}

// Flat stream: each array as count 16-byte packs, UNROLL packs per lane and trip at a
// stride of the whole grid, grid-stride loop.
template <int NIN, int UNROLL>
__global__ void __launch_bounds__(kMaxThreads) far_ceiling_flat_kernel(const StreamArgs a) {
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t bytes = a.count * 16;  // below 2^32 (checked on the host)
  const uint32_t nb = static_cast<uint32_t>(bytes);
  const bool half = a.out2_half != 0;
  __amdgpu_buffer_rsrc_t r[NIN];
#pragma unroll
  for (int i = 0; i < NIN; ++i) r[i] = rsrc(a.in[i], 0, nb);
  const __amdgpu_buffer_rsrc_t o1 = rsrc(a.out_full, 0, nb);
  const __amdgpu_buffer_rsrc_t o2 =
      rsrc(a.out2 != nullptr ? a.out2 : a.out_full, 0, a.out2 != nullptr ? (half ? nb / 2 : nb) : 0u);
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; base < a.count;
       base += nthreads * UNROLL) {
    uint32_t voff[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t o = (base + u * nthreads) * 16;
      voff[u] = static_cast<uint32_t>(o < bytes ? o : bytes);  // past the end: range check
    }
    u32x4 v[NIN][UNROLL];
#pragma unroll
    for (int i = 0; i < NIN; ++i)
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) v[i][u] = __builtin_amdgcn_raw_buffer_load_b128(r[i], voff[u], 0, kNonTemporal);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      u32x4 x = v[0][u];
#pragma unroll
      for (int i = 1; i < NIN; ++i) x ^= v[i][u];
      store_pack(x, o1, o2, half, voff[u]);
    }
  }
}

__global__ void far_ceiling_empty_kernel() {}

__global__ void __launch_bounds__(kWave) far_ceiling_sleep_kernel(int iterations) {
  for (int i = 0; i < iterations; ++i) __builtin_amdgcn_s_sleep(127);
}

__global__ void __launch_bounds__(kWave) far_ceiling_stamp_kernel(uint64_t* out, int index) {
  if (threadIdx.x == 0) out[index] = __builtin_amdgcn_s_memrealtime();
}

using Fn = void (*)(StreamArgs);

template <int NIN, int N>
constexpr Fn rows_fn() {
  if constexpr (NIN * N <= kMaxLoads) return &far_ceiling_rows_kernel<NIN, N>;
  else return nullptr;
}
template <int NIN, int N>
constexpr Fn flat_fn() {
  if constexpr (NIN * N <= kMaxLoads) return &far_ceiling_flat_kernel<NIN, N>;
  else return nullptr;
}

template <bool ROWS, int NIN, int... N>
constexpr std::array<Fn, sizeof...(N)> table_row(std::integer_sequence<int, N...>) {
  if constexpr (ROWS) return {{rows_fn<NIN, N + 1>()...}};
  else return {{flat_fn<NIN, N + 1>()...}};
}
template <bool ROWS, int... I>
constexpr std::array<std::array<Fn, kMaxPacks>, sizeof...(I)> table(std::integer_sequence<int, I...>) {
  return {{table_row<ROWS, I + 1>(std::make_integer_sequence<int, kMaxPacks>{})...}};
}
const auto kRows = table<true>(std::make_integer_sequence<int, kMaxIn>{});
const auto kFlat = table<false>(std::make_integer_sequence<int, kMaxIn>{});

int launch(Fn fn, int64_t grid, int block, const StreamArgs& a, far_ceiling_stream_t stream) {
  StreamArgs args = a;
  void* params[] = {&args};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<unsigned>(grid)),
                                       dim3(static_cast<unsigned>(block)), params, 0,
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 2;
}

bool fill_inputs(StreamArgs* a, const void* const* inputs, int n_inputs) {
  if (inputs == nullptr || n_inputs < 1 || n_inputs > kMaxIn) return false;
  for (int i = 0; i < n_inputs; ++i) {
    if (inputs[i] == nullptr) return false;
    a->in[i] = inputs[i];
  }
  return true;
}

}  // namespace

extern "C" {

int far_ceiling_rows(const void* const* inputs, int n_inputs, void* out_full, void* out2, int out2_half,
                     float* out_row, int64_t rows, int64_t row_bytes, int waves_per_row,
                     int packs_per_lane, int rows_per_block, int64_t grid_blocks,
                     far_ceiling_stream_t stream) {
  StreamArgs a = {};
  if (!fill_inputs(&a, inputs, n_inputs) || out_full == nullptr) return 1;
  if (rows < 1 || row_bytes < 16 || row_bytes % 16 != 0 || row_bytes >= (int64_t{1} << 31)) return 1;
  if (waves_per_row < 1 || rows_per_block < 1 || packs_per_lane < 1 || packs_per_lane > kMaxPacks) return 1;
  const int64_t block = int64_t{waves_per_row} * kWave * rows_per_block;
  if (block > kMaxThreads) return 1;
  if (int64_t{packs_per_lane} * waves_per_row * kWave * 16 < row_bytes) return 1;  // row must fit
  if (grid_blocks < 1 || grid_blocks > kMaxGrid) return 1;
  const Fn fn = kRows[n_inputs - 1][packs_per_lane - 1];
  if (fn == nullptr) return 1;
  a.out_full = out_full;
  a.out2 = out2;
  a.out2_half = out2_half != 0;
  a.out_row = out_row;
  a.count = rows;
  a.row_bytes = static_cast<int32_t>(row_bytes);
  a.waves_per_row = waves_per_row;
  a.rows_per_block = rows_per_block;
  return launch(fn, grid_blocks, static_cast<int>(block), a, stream);
}

int far_ceiling_flat(const void* const* inputs, int n_inputs, void* out_full, void* out2, int out2_half,
                     int64_t bytes, int unroll, int block_threads, int64_t grid_blocks,
                     far_ceiling_stream_t stream) {
  StreamArgs a = {};
  if (!fill_inputs(&a, inputs, n_inputs) || out_full == nullptr) return 1;
  if (bytes < 16 || bytes % 16 != 0 || bytes >= (int64_t{1} << 32)) return 1;
  if (unroll < 1 || unroll > kMaxPacks) return 1;
  if (block_threads < kWave || block_threads > kMaxThreads || block_threads % kWave != 0) return 1;
  if (grid_blocks < 1 || grid_blocks > kMaxGrid) return 1;
  const Fn fn = kFlat[n_inputs - 1][unroll - 1];
  if (fn == nullptr) return 1;
  a.out_full = out_full;
  a.out2 = out2;
  a.out2_half = out2_half != 0;
  a.count = bytes / 16;
  return launch(fn, grid_blocks, block_threads, a, stream);
}

int far_ceiling_empty(int64_t grid_blocks, int block_threads, far_ceiling_stream_t stream) {
  if (grid_blocks < 1 || grid_blocks > kMaxGrid) return 1;
  if (block_threads < kWave || block_threads > kMaxThreads || block_threads % kWave != 0) return 1;
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&far_ceiling_empty_kernel),
                                       dim3(static_cast<unsigned>(grid_blocks)),
                                       dim3(static_cast<unsigned>(block_threads)), nullptr, 0,
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 2;
}

int far_ceiling_sleep(int iterations, far_ceiling_stream_t stream) {
  if (iterations < 0 || iterations > 100000) return 1;
  void* params[] = {&iterations};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&far_ceiling_sleep_kernel), dim3(1),
                                       dim3(kWave), params, 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 2;
}

int far_ceiling_stamp(uint64_t* out, int index, far_ceiling_stream_t stream) {
  if (out == nullptr || index < 0) return 1;
  void* params[] = {&out, &index};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&far_ceiling_stamp_kernel), dim3(1),
                                       dim3(kWave), params, 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
