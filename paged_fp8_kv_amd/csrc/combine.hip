// Merge of the split partials and the gated output norm: a = (sum_s o_s 2^(m_s-M))
// / (sum_s l_s 2^(m_s-M)) * kv_scale, then out = rmsnorm(a) * w_o * sigmoid(gate)
// per head in bf16 (task page "Gated attention decode", section "What to
// compute", last line of the listing; output shape from the same section).
//
// One wave per (token, head); lane d owns output dim d.
#include "device_common.h"
#include "launch.h"

namespace museattn {

__global__ __launch_bounds__(64) void combine_kernel(StepArgs a) {
  const int th = blockIdx.x;          // t * 16 + h
  const int t = th / HQ, h = th % HQ;
  const int d = threadIdx.x;
  const int b = t / a.L;
  const KeyRange r = request_range(a, b);
  const int ns = valid_splits(a, r);
  const float *ml = a.part_ml + (size_t)th * a.nsplit * 2;
  const float *po = a.part_o + (size_t)th * a.nsplit * D;

  float M = -INFINITY;
  for (int s = d; s < ns; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));

  float lsum = 0.0f, o = 0.0f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int s = 0; s < ns; ++s) {
      const float ms = ml[2 * s];
      const float sc = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
      lsum += sc * ml[2 * s + 1];
      o += sc * po[(size_t)s * D + d];
    }
  }
  const float av = lsum > 0.0f ? o / lsum * a.kv_scale : 0.0f;
  const float ms2 = wave_sum(av * av) * (1.0f / 64.0f);
  const float y = av / sqrtf(ms2 + a.eps) * a.wo[d];
  const float g = bf16_bits_to_f32(a.qkv[(size_t)t * QKV_W + G_OFF + h * D + d]);
  const float gated = y / (1.0f + expf(-g));
  a.out[(size_t)t * (HQ * D) + h * D + d] = f32_to_bf16_bits(gated);
}

void launch_combine(const StepArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.B * a.L * HQ), dim3(64), 0, stream, a);
}

}  // namespace museattn
