// far_api.hip -- the C ABI (include/far.h): argument validation, the token-count-aware
// launch plan and the dispatch to the kernel instantiations.
//
// Validation happens before any HIP call, so every error path can be exercised on a
// machine without a GPU. Nothing here allocates, synchronises or keeps a pointer; the
// only process-wide state is the FAR_LOG switch, read once.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "far.h"
#include "far_launch.hpp"

namespace {

constexpr int64_t kMaxHidden = int64_t{1} << 30;
constexpr int64_t kMaxTokens = 0x7fffffff;
// Launch-plan constants (see auto_plan).
constexpr int64_t kDecodeWaves = 4096;       // rows x waves at one pack per lane, at most
constexpr int64_t kDecodeMaxWaves = 8;       // waves per row in the decode regime
constexpr int64_t kPrefillPacksPerLane = 2;     // prefill: packs per lane (at least)
constexpr int kPrefillEvenTeamPartials = 5;     // from this P, prefer an even team (see auto_plan)
constexpr int64_t kPrefillShortRowsPerBlock = 8; // prefill rows of at most 64 packs
constexpr int64_t kResidentWaves = 32 * 256;    // waves the chip holds at once (32 per CU)
constexpr int kScaleThreads = 1024;          // per-tensor scale reduction (one workgroup)
// Workgroups per launch, at most. A dispatch covers fewer than 2^32 work-items (its
// grid size is a 32-bit count), so very large T with short rows cannot give every row
// its own team; both kernels loop over rows when the grid is smaller than the batch.
// 2^20 workgroups of <= 1024 lanes stay below that limit and far above what fills the
// chip.
constexpr int64_t kMaxGridBlocks = int64_t{1} << 20;
constexpr int64_t kQuantMaxBlocks = 16384;   // per-tensor code pass (grid-stride)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FAR_LOG set to anything but "" or "0": one line per call on stderr with the shape and
// the launch plan (read once per process).
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("FAR_LOG");
    return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
  }();
  return on;
}

far_status_t check_scalars(int64_t T, int64_t H, int P, far_dtype_t dtype, far_quant_t quant) {
  if (P < 1 || P > FAR_MAX_PARTIALS) return FAR_ERR_BAD_NUM_PARTIALS;
  if (dtype != FAR_DTYPE_BF16 && dtype != FAR_DTYPE_FP16) return FAR_ERR_BAD_DTYPE;
  if (quant != FAR_QUANT_NONE && quant != FAR_QUANT_FP8_STATIC_TENSOR &&
      quant != FAR_QUANT_FP8_DYNAMIC_TOKEN && quant != FAR_QUANT_FP8_DYNAMIC_GROUP &&
      quant != FAR_QUANT_FP8_DYNAMIC_TENSOR)
    return FAR_ERR_BAD_QUANT_ARGS;
  if (T < 0 || T > kMaxTokens || H < 1 || H > kMaxHidden) return FAR_ERR_BAD_SHAPE;
  return FAR_OK;
}

static_assert(FAR_MAX_WAVES_PER_ROW == far::kMaxWavesPerBlock, "far.h and the kernels disagree");
static_assert(FAR_MAX_PACKS_PER_LANE == far::kMaxPacksPerLane, "far.h and the kernels disagree");
static_assert(FAR_FP8_GROUP == far::kFp8Group, "far.h and the kernels disagree");
static_assert(static_cast<int>(FAR_QUANT_FP8_DYNAMIC_GROUP) == far::kQuantDynamicGroup &&
                  static_cast<int>(FAR_QUANT_FP8_DYNAMIC_TENSOR) == far::kQuantDynamicTensor,
              "far.h and the kernels disagree");

int64_t workspace_need(int64_t T, far_quant_t quant) {
  return quant == FAR_QUANT_FP8_DYNAMIC_TENSOR ? 8 * T : 0;
}

}  // namespace

// Scratch of far_fused_add_rmsnorm_noalloc: the workspace of the per-tensor mode (per-row
// max |y| and r) for callers that cannot allocate. Each GPU holds its own copy from
// the library's load until the process ends. In host code `scratch` names a host-side
// stand-in, never the device memory: kernels get the address that hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char scratch[FAR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept. nullptr with *err set if the runtime fails.
void* scratch_on_current_device(hipError_t* err) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

// Largest row the vector variant holds in registers: 16 waves x 64 lanes x 5 packs.
constexpr int64_t kMaxVectorPacks =
    int64_t{far::kMaxWavesPerBlock} * far::kWave * far::kMaxPacksPerLane;

// One workgroup per row, with about kGenUnroll elements per lane (64..1024 lanes).
void generic_plan(int64_t T, int64_t H, far_plan_t* p) {
  int64_t lanes = cdiv(cdiv(H, far::kGenUnroll), far::kWave) * far::kWave;
  if (lanes > far::kGenMaxThreads) lanes = far::kGenMaxThreads;
  p->variant = FAR_VARIANT_GENERIC;
  p->waves_per_row = static_cast<int32_t>(lanes / far::kWave);
  p->rows_per_block = 1;
  p->packs_per_lane = 0;
  p->block_threads = static_cast<int32_t>(lanes);
  p->grid_blocks = T < kMaxGridBlocks ? T : kMaxGridBlocks;
}

// The automatic plan. packs = ceil(H / 8) 16-byte packs per row (the last one partial
// when H % 8 != 0). Measured on MI355X:
//  - decode (few rows: the batch cannot fill the chip even at one pack per lane):
//    spread each row over up to 8 waves, one workgroup per row, so the rows cover as
//    many CUs as they can; teams of 16 waves cost more in the cross-wave reduction
//    than they gain;
//  - prefill (many rows): one row per workgroup, two packs per lane (the fewest waves
//    that hold the row that way), which beat several rows per workgroup with deeper
//    lanes by 2% on average over 106 prefill shapes (P 1-8, H 512-16384, T 2048-16384,
//    bf16 and fp16, with and without fp8), by 4% on P = 2 [2048, 5120] with dynamic fp8;
//    with five or more partials, an odd team at two packs (18+ loads per lane, so few
//    waves per SIMD) takes three packs instead when that gives an even team (P = 8,
//    H = 5120: 4 x 3 is 11-15% faster than 5 x 2). A grid of one row per workgroup that
//    would need between one and one and a half rounds of the chip's resident waves (32
//    per CU) leaves its last round mostly empty; those batches take half as many
//    workgroups, each looping over two rows (over 96 shapes with T 2048-6144, looping
//    beyond 1.5 rounds lost as often as it gained). Rows that fit one pack per lane (at
//    most 64 packs) keep eight rows per workgroup.
void auto_plan(int64_t T, int64_t H, int P, far_quant_t quant, bool vector_ok, far_plan_t* p) {
  std::memset(p, 0, sizeof(*p));
  if (T == 0) {
    p->variant = FAR_VARIANT_EMPTY;
    return;
  }
  const int64_t packs = cdiv(H, 8);
  if (!vector_ok || packs > kMaxVectorPacks) {
    generic_plan(T, H, p);
    return;
  }
  const int64_t kMaxW = far::kMaxWavesPerBlock;
  const int64_t kMaxN = far::max_packs_for(static_cast<int>(quant));
  if (packs > kMaxW * far::kWave * kMaxN) {
    generic_plan(T, H, p);
    return;
  }
  const int64_t waves_at_one_pack = T * (cdiv(packs, far::kWave) < kMaxW ? cdiv(packs, far::kWave) : kMaxW);
  int64_t wpr, npack, rpb, trips = 1;
  if (waves_at_one_pack <= kDecodeWaves) {
    npack = cdiv(packs, far::kWave * kDecodeMaxWaves);
    if (npack > kMaxN) npack = kMaxN;
    if (npack < cdiv(packs, far::kWave * kMaxW)) npack = cdiv(packs, far::kWave * kMaxW);
    if (npack < 1) npack = 1;
    wpr = cdiv(packs, far::kWave * npack);
    rpb = 1;
  } else {
    npack = kPrefillPacksPerLane;
    if (npack < cdiv(packs, far::kWave * kMaxW)) npack = cdiv(packs, far::kWave * kMaxW);
    wpr = cdiv(packs, far::kWave * npack);
    if (P >= kPrefillEvenTeamPartials && wpr > 1 && wpr % 2 == 1 && npack < kMaxN &&
        cdiv(packs, far::kWave * (npack + 1)) % 2 == 0)
      wpr = cdiv(packs, far::kWave * (npack + 1));
    if (packs <= far::kWave) {
      rpb = kPrefillShortRowsPerBlock;
    } else {
      rpb = wpr == 1 ? 2 : 1;
      const int64_t waves = T * wpr;
      if (waves > kResidentWaves && 2 * waves <= 3 * kResidentWaves) trips = 2;
    }
  }
  npack = cdiv(packs, far::kWave * wpr);  // shallowest depth for this team size
  const int64_t groups = cdiv(T, rpb);
  const int64_t grid = cdiv(groups, trips);
  p->variant = FAR_VARIANT_VECTOR;
  p->waves_per_row = static_cast<int32_t>(wpr);
  p->packs_per_lane = static_cast<int32_t>(npack);
  p->rows_per_block = static_cast<int32_t>(rpb);
  p->block_threads = static_cast<int32_t>(rpb * wpr * far::kWave);
  p->grid_blocks = grid < kMaxGridBlocks ? grid : kMaxGridBlocks;
}

far_status_t check_plan(int64_t T, int64_t H, far_quant_t quant, bool vector_ok, far_plan_t* p) {
  if (T == 0) {
    std::memset(p, 0, sizeof(*p));
    p->variant = FAR_VARIANT_EMPTY;
    return FAR_OK;
  }
  if (p->variant == FAR_VARIANT_GENERIC) {
    generic_plan(T, H, p);
    return FAR_OK;
  }
  if (p->variant != FAR_VARIANT_VECTOR) return FAR_ERR_BAD_PLAN;
  if (!vector_ok) return FAR_ERR_BAD_PLAN;
  const int64_t packs = cdiv(H, 8);
  if (p->waves_per_row < 1 || p->waves_per_row > far::kMaxWavesPerBlock) return FAR_ERR_BAD_PLAN;
  if (p->packs_per_lane < 1 || p->packs_per_lane > far::max_packs_for(static_cast<int>(quant)))
    return FAR_ERR_BAD_PLAN;
  if (p->rows_per_block < 1) return FAR_ERR_BAD_PLAN;
  const int64_t block = int64_t{p->rows_per_block} * p->waves_per_row * far::kWave;
  if (block > far::kVecMaxThreads) return FAR_ERR_BAD_PLAN;
  if (int64_t{p->packs_per_lane} * p->waves_per_row * far::kWave < packs) return FAR_ERR_BAD_PLAN;
  p->block_threads = static_cast<int32_t>(block);
  // fewer workgroups than row groups: each team loops over rows (grid-stride)
  const int64_t groups = cdiv(T, p->rows_per_block);
  if (p->grid_blocks < 0) return FAR_ERR_BAD_PLAN;
  if (p->grid_blocks == 0 || p->grid_blocks > groups) p->grid_blocks = groups;
  if (p->grid_blocks > kMaxGridBlocks) p->grid_blocks = kMaxGridBlocks;
  return FAR_OK;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  const uintptr_t y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

bool aligned(const void* p, uintptr_t n) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

struct Span {
  const void* p;
  int64_t n;
  bool row_tensor;  // a [T, H] input that residual_out may coincide with exactly
};

// Where the per-tensor mode's workspace comes from: the caller's argument, or the
// library's per-device scratch array (far_fused_add_rmsnorm_noalloc).
enum class WorkspaceSource { kArgument, kScratch };

far_status_t run(const void* const* partials, int P, const void* residual, const void* gamma,
                 int64_t T, int64_t H, far_dtype_t dtype, float eps, float weight_bias,
                 far_quant_t quant, const float* scale, void* norm_out, void* residual_out,
                 void* quant_out, float* scale_out, far_stream_t stream,
                 const far_plan_t* forced, void* workspace, int64_t workspace_bytes,
                 WorkspaceSource ws_source = WorkspaceSource::kArgument) {
  far_status_t st = check_scalars(T, H, P, dtype, quant);
  if (st != FAR_OK) return st;
  if (partials == nullptr) return FAR_ERR_NULL_POINTER;
  if (T == 0) return FAR_OK;  // nothing to read or write

  for (int p = 0; p < P; ++p)
    if (partials[p] == nullptr) return FAR_ERR_NULL_POINTER;
  // residual NULL: the form without a residual input (new residual = sum of partials);
  // residual_out NULL: the new residual is not written
  if (gamma == nullptr) return FAR_ERR_NULL_POINTER;
  switch (quant) {
    case FAR_QUANT_NONE:
      if (norm_out == nullptr) return FAR_ERR_NULL_POINTER;
      if (scale != nullptr || quant_out != nullptr || scale_out != nullptr)
        return FAR_ERR_BAD_QUANT_ARGS;
      break;
    case FAR_QUANT_FP8_STATIC_TENSOR:
      if (scale == nullptr || quant_out == nullptr || scale_out != nullptr)
        return FAR_ERR_BAD_QUANT_ARGS;
      break;
    case FAR_QUANT_FP8_DYNAMIC_TOKEN:
    case FAR_QUANT_FP8_DYNAMIC_GROUP:
    case FAR_QUANT_FP8_DYNAMIC_TENSOR:
      if (scale != nullptr || quant_out == nullptr || scale_out == nullptr)
        return FAR_ERR_BAD_QUANT_ARGS;
      break;
  }
  const int64_t ws_need = workspace_need(T, quant);
  if (ws_source == WorkspaceSource::kScratch) {
    // the scratch array is the workspace: its size is the limit, and being a separate
    // allocation of the library it overlaps no caller tensor
    if (ws_need > FAR_NOALLOC_SCRATCH_BYTES) return FAR_ERR_SCRATCH_LIMIT;
    workspace = nullptr;
  } else if (ws_need > 0 && (workspace == nullptr || workspace_bytes < ws_need)) {
    return FAR_ERR_WORKSPACE;
  }

  // ---- aliasing
  const int64_t e = 2;
  const int64_t tensor = T * H * e;
  Span inputs[FAR_MAX_PARTIALS + 3];
  int n_in = 0;
  for (int p = 0; p < P; ++p) inputs[n_in++] = {partials[p], tensor, true};
  if (residual != nullptr) inputs[n_in++] = {residual, tensor, true};
  inputs[n_in++] = {gamma, H * e, false};
  if (scale != nullptr) inputs[n_in++] = {scale, 4, false};
  // residual_out: each element of a row tensor is read by the lane that writes it, so
  // residual_out may coincide exactly with the residual (in-place update) or with a
  // partial's buffer. gamma and the static scale are read by every row, so writing
  // over them is a race even when the sizes match (T == 1 makes gamma as large as a
  // row tensor); any other overlap is a race too.
  for (int i = 0; residual_out != nullptr && i < n_in; ++i) {
    const bool same_tensor = inputs[i].row_tensor && inputs[i].p == residual_out;
    if (!same_tensor && overlaps(inputs[i].p, inputs[i].n, residual_out, tensor))
      return FAR_ERR_BAD_ALIAS;
  }
  // the other outputs overlap nothing
  const int64_t groups = cdiv(H, far::kFp8Group);
  const int64_t scale_elems = quant == FAR_QUANT_FP8_DYNAMIC_TOKEN ? T
                            : quant == FAR_QUANT_FP8_DYNAMIC_GROUP ? T * groups
                            : 1;
  // the other outputs and the workspace overlap nothing
  const Span outs[4] = {{norm_out, norm_out ? tensor : 0, false},
                        {quant_out, quant_out ? T * H : 0, false},
                        {scale_out, scale_out ? 4 * scale_elems : 0, false},
                        {ws_need > 0 ? workspace : nullptr, ws_need, false}};
  for (int o = 0; o < 4; ++o) {
    if (outs[o].p == nullptr) continue;
    for (int i = 0; i < n_in; ++i)
      if (overlaps(inputs[i].p, inputs[i].n, outs[o].p, outs[o].n)) return FAR_ERR_BAD_ALIAS;
    if (overlaps(residual_out, tensor, outs[o].p, outs[o].n)) return FAR_ERR_BAD_ALIAS;
    for (int q = o + 1; q < 4; ++q)
      if (overlaps(outs[q].p, outs[q].n, outs[o].p, outs[o].n)) return FAR_ERR_BAD_ALIAS;
  }

  // ---- variant
  // The vector kernels need element alignment only: gfx950 serves 16-byte accesses at
  // any address (the compiler itself emits them for unaligned copies), so e.g. a view
  // starting one element into a buffer stays fast. Rows with H % 8 != 0 take the
  // kernels' partial-last-pack form.
  bool vector_ok = true;
  for (int p = 0; p < P; ++p) vector_ok = vector_ok && aligned(partials[p], 2);
  vector_ok = vector_ok && aligned(residual, 2) && aligned(gamma, 2) &&
              aligned(residual_out, 2) && aligned(norm_out, 2);

  far_plan_t plan;
  if (forced != nullptr) {
    plan = *forced;
    st = check_plan(T, H, quant, vector_ok, &plan);
    if (st != FAR_OK) return st;
  } else {
    auto_plan(T, H, P, quant, vector_ok, &plan);
  }

  // prefill-sized batches (the plan's regime test) store the new residual through the
  // cache; decode-sized kernels would end waiting for its write-back
  const bool cached_residual = plan.variant == FAR_VARIANT_VECTOR &&
                               T * cdiv(cdiv(H, 8), far::kWave) > kDecodeWaves;

  if (log_enabled()) {
    static const char* const kQuantNames[] = {"none", "static", "dynamic", "group", "tensor"};
    std::fprintf(stderr,
                 "far: T=%lld H=%lld P=%d %s quant=%s residual=%s residual_out=%s -> %s "
                 "waves_per_row=%d packs_per_lane=%d rows_per_block=%d block=%d grid=%lld "
                 "residual_stores=%s\n",
                 static_cast<long long>(T), static_cast<long long>(H), P,
                 dtype == FAR_DTYPE_BF16 ? "bf16" : "fp16", kQuantNames[quant],
                 residual != nullptr ? "yes" : "no", residual_out != nullptr ? "yes" : "no",
                 plan.variant == FAR_VARIANT_VECTOR ? "vector" : "generic", plan.waves_per_row,
                 plan.packs_per_lane, plan.rows_per_block, plan.block_threads,
                 static_cast<long long>(plan.grid_blocks), cached_residual ? "cached" : "streamed");
  }

  if (ws_need > 0 && ws_source == WorkspaceSource::kScratch) {
    // after every validation: the first call on a device looks the address up
    hipError_t e = hipSuccess;
    workspace = scratch_on_current_device(&e);
    if (workspace == nullptr) return FAR_ERR_HIP;
  }

  far::KernelArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int p = 0; p < P; ++p) a.partials[p] = partials[p];
  a.residual = residual;
  a.gamma = gamma;
  a.residual_out = residual_out;
  a.norm_out = norm_out;
  a.quant_out = static_cast<uint8_t*>(quant_out);
  a.scale_out = scale_out;
  a.scale = scale;
  a.workspace = static_cast<float*>(ws_need > 0 ? workspace : nullptr);
  a.num_tokens = T;
  a.hidden = static_cast<int32_t>(H);
  a.num_partials = P;
  a.groups = static_cast<int32_t>(groups);
  a.eps = eps;
  a.weight_bias = weight_bias;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  const dim3 grid(static_cast<unsigned>(plan.grid_blocks));
  const bool bf = dtype == FAR_DTYPE_BF16;
  if (plan.variant == FAR_VARIANT_VECTOR) {
    const dim3 block(static_cast<unsigned>(plan.block_threads));
    const int n = plan.packs_per_lane, w = plan.waves_per_row, r = plan.rows_per_block;
    const bool cached = cached_residual;
#define FAR_VEC(D, Q) far::launch_vector_##D##_##Q(P, n, grid, block, a, w, r, cached, s)
    switch (quant) {
      case FAR_QUANT_NONE: err = bf ? FAR_VEC(bf16, none) : FAR_VEC(fp16, none); break;
      case FAR_QUANT_FP8_STATIC_TENSOR: err = bf ? FAR_VEC(bf16, static) : FAR_VEC(fp16, static); break;
      case FAR_QUANT_FP8_DYNAMIC_TOKEN: err = bf ? FAR_VEC(bf16, dynamic) : FAR_VEC(fp16, dynamic); break;
      case FAR_QUANT_FP8_DYNAMIC_GROUP: err = bf ? FAR_VEC(bf16, group) : FAR_VEC(fp16, group); break;
      case FAR_QUANT_FP8_DYNAMIC_TENSOR: err = bf ? FAR_VEC(bf16, tensor) : FAR_VEC(fp16, tensor); break;
    }
#undef FAR_VEC
  } else {
    const dim3 block(static_cast<unsigned>(plan.block_threads));
#define FAR_GEN(D, Q) far::launch_generic_##D##_##Q(P, grid, block, a, s)
    switch (quant) {
      case FAR_QUANT_NONE: err = bf ? FAR_GEN(bf16, none) : FAR_GEN(fp16, none); break;
      case FAR_QUANT_FP8_STATIC_TENSOR: err = bf ? FAR_GEN(bf16, static) : FAR_GEN(fp16, static); break;
      case FAR_QUANT_FP8_DYNAMIC_TOKEN: err = bf ? FAR_GEN(bf16, dynamic) : FAR_GEN(fp16, dynamic); break;
      case FAR_QUANT_FP8_DYNAMIC_GROUP: err = bf ? FAR_GEN(bf16, group) : FAR_GEN(fp16, group); break;
      case FAR_QUANT_FP8_DYNAMIC_TENSOR: err = bf ? FAR_GEN(bf16, tensor) : FAR_GEN(fp16, tensor); break;
    }
#undef FAR_GEN
  }
  if (err == hipSuccess && quant == FAR_QUANT_FP8_DYNAMIC_TENSOR) {
    // tensor scale from the per-row maxima, then the codes
    const float* row_max = a.workspace;
    void* sp[] = {const_cast<float**>(&row_max), &a.num_tokens, &a.scale_out};
    err = hipLaunchKernel(reinterpret_cast<const void*>(&far::far_tensor_scale_kernel<kScaleThreads>),
                          dim3(1), dim3(kScaleThreads), sp, 0, s);
    if (err == hipSuccess) {
      // packs of 8 codes (a row's partial last pack element by element) after the vector
      // kernels, one code per lane and step after the generic kernel
      const bool vec = plan.variant == FAR_VARIANT_VECTOR;
      const int64_t units = T * (vec ? cdiv(H, 8) : H);
      int64_t blocks = cdiv(units, far::kQuantThreads);
      if (blocks > kQuantMaxBlocks) blocks = kQuantMaxBlocks;
      void* qp[] = {&a};
      const void* fn = bf ? (vec ? reinterpret_cast<const void*>(&far::far_tensor_quant_kernel<far::Bf16, true>)
                                 : reinterpret_cast<const void*>(&far::far_tensor_quant_kernel<far::Bf16, false>))
                          : (vec ? reinterpret_cast<const void*>(&far::far_tensor_quant_kernel<far::Fp16, true>)
                                 : reinterpret_cast<const void*>(&far::far_tensor_quant_kernel<far::Fp16, false>));
      err = hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(far::kQuantThreads), qp, 0, s);
    }
  }
  return err == hipSuccess ? FAR_OK : FAR_ERR_HIP;
}

}  // namespace

extern "C" {

far_status_t far_fused_add_rmsnorm(const void* const* partials, int num_partials,
                                   const void* residual, const void* gamma, int64_t num_tokens,
                                   int64_t hidden, far_dtype_t dtype, float eps,
                                   float weight_bias, far_quant_t quant_mode, const float* scale,
                                   void* norm_out, void* residual_out, void* quant_out,
                                   float* scale_out, far_stream_t stream) {
  return run(partials, num_partials, residual, gamma, num_tokens, hidden, dtype, eps,
             weight_bias, quant_mode, scale, norm_out, residual_out, quant_out, scale_out,
             stream, nullptr, nullptr, 0);
}

far_status_t far_fused_add_rmsnorm_ex(
    const void* const* partials, int num_partials, const void* residual, const void* gamma,
    int64_t num_tokens, int64_t hidden, far_dtype_t dtype, float eps, float weight_bias,
    far_quant_t quant_mode, const float* scale, void* norm_out, void* residual_out,
    void* quant_out, float* scale_out, far_stream_t stream, const far_plan_t* plan,
    void* workspace, int64_t workspace_bytes) {
  return run(partials, num_partials, residual, gamma, num_tokens, hidden, dtype, eps,
             weight_bias, quant_mode, scale, norm_out, residual_out, quant_out, scale_out,
             stream, plan, workspace, workspace_bytes);
}

far_status_t far_fused_add_rmsnorm_noalloc(const void* const* partials, int num_partials,
                                           const void* residual, const void* gamma,
                                           int64_t num_tokens, int64_t hidden, far_dtype_t dtype,
                                           float eps, float weight_bias, far_quant_t quant_mode,
                                           const float* scale, void* norm_out, void* residual_out,
                                           void* quant_out, float* scale_out, far_stream_t stream) {
  return run(partials, num_partials, residual, gamma, num_tokens, hidden, dtype, eps,
             weight_bias, quant_mode, scale, norm_out, residual_out, quant_out, scale_out,
             stream, nullptr, nullptr, 0, WorkspaceSource::kScratch);
}

int64_t far_workspace_bytes(int64_t num_tokens, int64_t hidden, far_quant_t quant_mode) {
  if (check_scalars(num_tokens, hidden, 1, FAR_DTYPE_BF16, quant_mode) != FAR_OK) return -1;
  return workspace_need(num_tokens, quant_mode);
}

far_status_t far_plan(int64_t num_tokens, int64_t hidden, int num_partials, far_dtype_t dtype,
                      far_quant_t quant_mode, far_plan_t* out) {
  if (out == nullptr) return FAR_ERR_NULL_POINTER;
  const far_status_t st = check_scalars(num_tokens, hidden, num_partials, dtype, quant_mode);
  if (st != FAR_OK) return st;
  auto_plan(num_tokens, hidden, num_partials, quant_mode, true, out);
  return FAR_OK;
}

const char* far_status_string(far_status_t status) {
  switch (status) {
    case FAR_OK: return "FAR_OK";
    case FAR_ERR_NULL_POINTER: return "FAR_ERR_NULL_POINTER: a required pointer is NULL";
    case FAR_ERR_BAD_SHAPE: return "FAR_ERR_BAD_SHAPE: num_tokens or hidden out of range";
    case FAR_ERR_BAD_DTYPE: return "FAR_ERR_BAD_DTYPE: unknown storage dtype";
    case FAR_ERR_BAD_NUM_PARTIALS: return "FAR_ERR_BAD_NUM_PARTIALS: num_partials not in [1, 8]";
    case FAR_ERR_BAD_QUANT_ARGS:
      return "FAR_ERR_BAD_QUANT_ARGS: quant mode and scale/quant_out/scale_out disagree";
    case FAR_ERR_BAD_ALIAS: return "FAR_ERR_BAD_ALIAS: an output overlaps another tensor";
    case FAR_ERR_HIP: return "FAR_ERR_HIP: the HIP runtime refused the launch";
    case FAR_ERR_BAD_PLAN: return "FAR_ERR_BAD_PLAN: the explicit plan does not fit the shape";
    case FAR_ERR_WORKSPACE: return "FAR_ERR_WORKSPACE: the mode needs a (larger) workspace";
    case FAR_ERR_SCRATCH_LIMIT:
      return "FAR_ERR_SCRATCH_LIMIT: the batch needs more scratch than the no-allocation entry "
             "point holds (per-tensor mode: 8 * num_tokens > FAR_NOALLOC_SCRATCH_BYTES)";
  }
  return "FAR_ERR_UNKNOWN: not a far_status_t value";
}

int far_version(void) { return 10000; }

}  // extern "C"
