// far_inst.hip -- instantiates the vector kernel for every (P, packs per lane) pair, in
// four forms (rows of whole packs, and rows ending in a partial pack, each with the new
// residual streamed out or stored through the cache), and the generic kernel for every P,
// for one (storage dtype, quant mode) given on the command line:
//   -DFAR_INST_DTYPE=bf16|fp16 -DFAR_INST_QUANT=none|static|dynamic|group|tensor
#include <array>
#include <utility>

#include "far_launch.hpp"

#ifndef FAR_INST_DTYPE
#error "define FAR_INST_DTYPE"
#endif
#ifndef FAR_INST_QUANT
#error "define FAR_INST_QUANT"
#endif

#define FAR_CAT3(a, b, c) a##_##b##_##c
#define FAR_NAME(base, d, q) FAR_CAT3(base, d, q)

namespace far {
namespace {

struct bf16_tag { using type = Bf16; };
struct fp16_tag { using type = Fp16; };
struct none_tag { static constexpr int value = kQuantNone; };
struct static_tag { static constexpr int value = kQuantStatic; };
struct dynamic_tag { static constexpr int value = kQuantDynamic; };
struct group_tag { static constexpr int value = kQuantDynamicGroup; };
struct tensor_tag { static constexpr int value = kQuantDynamicTensor; };

#define FAR_TAG(x) FAR_TAG2(x)
#define FAR_TAG2(x) x##_tag
using Fmt = FAR_TAG(FAR_INST_DTYPE)::type;
constexpr int kQuant = FAR_TAG(FAR_INST_QUANT)::value;

using VecFn = void (*)(KernelArgs, int, int);

// Depths a mode does not support (max_packs_for) have no kernel.
template <bool R, bool C, int P, int N>
constexpr VecFn vec_fn() {
  if constexpr (N <= max_packs_for(kQuant)) return &far_vec_kernel<Fmt, P, N, kQuant, R, C>;
  else return nullptr;
}

template <bool R, bool C, int P, int... N>
constexpr std::array<VecFn, sizeof...(N)> row_of(std::integer_sequence<int, N...>) {
  return {{vec_fn<R, C, P, N + 1>()...}};
}

template <bool R, bool C, int... P>
constexpr std::array<std::array<VecFn, kMaxPacksPerLane>, sizeof...(P)> table_of(
    std::integer_sequence<int, P...>) {
  return {{row_of<R, C, P + 1>(std::make_integer_sequence<int, kMaxPacksPerLane>{})...}};
}

// [0]: rows of whole packs (H % 8 == 0); [1]: rows ending in a partial pack; [2], [3]: the
// same with the new residual stored with the default cache policy (prefill)
const std::array<std::array<std::array<VecFn, kMaxPacksPerLane>, kMaxPartials>, 4> kVecTable = {
    {table_of<false, false>(std::make_integer_sequence<int, kMaxPartials>{}),
     table_of<true, false>(std::make_integer_sequence<int, kMaxPartials>{}),
     table_of<false, true>(std::make_integer_sequence<int, kMaxPartials>{}),
     table_of<true, true>(std::make_integer_sequence<int, kMaxPartials>{})}};

using GenFn = void (*)(KernelArgs);

template <int... P>
constexpr std::array<GenFn, sizeof...(P)> gen_table_of(std::integer_sequence<int, P...>) {
  return {{&far_generic_kernel<Fmt, P + 1, kQuant>...}};
}

const auto kGenTable = gen_table_of(std::make_integer_sequence<int, kMaxPartials>{});

}  // namespace

hipError_t FAR_NAME(launch_vector, FAR_INST_DTYPE, FAR_INST_QUANT)(
    int num_partials, int packs_per_lane, dim3 grid, dim3 block, const KernelArgs& a,
    int waves_per_row, int rows_per_block, bool cached_residual, hipStream_t stream) {
  if (num_partials < 1 || num_partials > kMaxPartials || packs_per_lane < 1 ||
      packs_per_lane > kMaxPacksPerLane)
    return hipErrorInvalidValue;
  const int form = (a.hidden % 8 != 0 ? 1 : 0) + (cached_residual ? 2 : 0);
  VecFn fn = kVecTable[form][num_partials - 1][packs_per_lane - 1];
  if (fn == nullptr) return hipErrorInvalidValue;
  KernelArgs args = a;
  int wpr = waves_per_row, rpb = rows_per_block;
  void* params[] = {&args, &wpr, &rpb};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, params, 0, stream);
}

hipError_t FAR_NAME(launch_generic, FAR_INST_DTYPE, FAR_INST_QUANT)(
    int num_partials, dim3 grid, dim3 block, const KernelArgs& a, hipStream_t stream) {
  if (num_partials < 1 || num_partials > kMaxPartials || block.x < kWave ||
      block.x > kGenMaxThreads || block.x % kWave != 0)
    return hipErrorInvalidValue;
  KernelArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(kGenTable[num_partials - 1]), grid, block,
                         params, 0, stream);
}

}  // namespace far
