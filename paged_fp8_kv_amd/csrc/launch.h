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
// the gather probe (a memory-system measurement, not part of the step)
void launch_gather_probe(const int32_t *table, const int32_t *seq_lens, const uint8_t *kc,
                         const uint8_t *vc, int B, int table_stride, int max_seq_len,
                         int page_size, int64_t num_rows, uint32_t *out, int work_groups,
                         hipStream_t stream);
}  // namespace museattn
