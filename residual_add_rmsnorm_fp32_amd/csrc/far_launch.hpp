// far_launch.hpp -- host-side launch entry points of the kernel instantiations.
// far_inst.hip is compiled once per (storage dtype, quant mode); each object defines
// the two functions below under a name carrying that pair. The per-tensor mode's
// second and third kernels are launched from far_api.hip.
#pragma once

#include <hip/hip_runtime.h>

#include "far_kernels.hpp"

namespace far {

#define FAR_DECLARE_LAUNCHERS(D, Q)                                                       \
  hipError_t launch_vector_##D##_##Q(int num_partials, int packs_per_lane, dim3 grid,     \
                                     dim3 block, const KernelArgs& a, int waves_per_row, \
                                     int rows_per_block, bool cached_residual,           \
                                     hipStream_t stream);                                 \
  hipError_t launch_generic_##D##_##Q(int num_partials, dim3 grid, dim3 block,            \
                                      const KernelArgs& a, hipStream_t stream);

FAR_DECLARE_LAUNCHERS(bf16, none)
FAR_DECLARE_LAUNCHERS(bf16, static)
FAR_DECLARE_LAUNCHERS(bf16, dynamic)
FAR_DECLARE_LAUNCHERS(fp16, none)
FAR_DECLARE_LAUNCHERS(fp16, static)
FAR_DECLARE_LAUNCHERS(fp16, dynamic)
FAR_DECLARE_LAUNCHERS(bf16, group)
FAR_DECLARE_LAUNCHERS(fp16, group)
FAR_DECLARE_LAUNCHERS(bf16, tensor)
FAR_DECLARE_LAUNCHERS(fp16, tensor)

#undef FAR_DECLARE_LAUNCHERS

}  // namespace far
