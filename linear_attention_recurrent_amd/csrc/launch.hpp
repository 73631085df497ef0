// Internal launchers (host side) for the DeltaLog kernels.  Arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include "dl_device.hpp"

namespace dl {

hipError_t launch_decode(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                         const StepArgs& s, hipStream_t stream);
hipError_t launch_merge(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                        int min_fill, hipStream_t stream);
hipError_t launch_merge_mfma(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                             int min_fill, hipStream_t stream);
hipError_t launch_init(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                       const float* init_base, hipStream_t stream);
hipError_t launch_prefill(int variant, bool bf16_base, int dk, int dv, int tiles, const PoolArgs& p,
                          const PrefillArgs& a, hipStream_t stream);
hipError_t launch_eager(int variant, int dk, int dv, int tiles, int heads, float* state, const StepArgs& s,
                        hipStream_t stream);

}  // namespace dl
