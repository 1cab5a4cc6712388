// Host-side launchers of the step's kernels (each defined next to its kernel).
#pragma once

#include "device_common.h"

namespace museattn {
void launch_attn(const StepArgs &a, hipStream_t stream);
void launch_combine(const StepArgs &a, hipStream_t stream);
void launch_rows(const StepArgs &a, hipStream_t stream);
void launch_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                  hipStream_t stream);
// the projection as an LDS-tiled MFMA GEMM (many tokens)
void gemm_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                hipStream_t stream);
}  // namespace museattn
