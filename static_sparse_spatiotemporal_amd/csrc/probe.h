// Launcher of the measured-MFMA-peak loop (probe.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tra {

// MFMA flops of one launch of `blocks` workgroups running `iters` rounds.
int64_t mfma_loop_flops(int64_t iters, int blocks);
hipError_t launch_mfma_loop(int64_t iters, int blocks, float *out, hipStream_t st);

}  // namespace tra
