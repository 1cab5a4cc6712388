// Prologue of the attention step: split of the fused projection row, QK-RMSNorm,
// RoPE on sliding-window layers, fp8 quantisation of the new k and v and their
// scatter into the paged cache (task page "Gated attention decode", section
// "What to compute", the first four lines of its listing).
//
// One wave per block token; lane d owns dimension d of every head, so each
// head's rmsnorm is one wave reduction and RoPE pairs (d, d ^ 32) are one lane
// swap.  The work is a few KB per token: the kernel is launch-latency bound.
#include "device_common.h"
#include "launch.h"

namespace museattn {

// E4M3FN byte of x (OCP format: bias 7, max 448, no infinities), round to
// nearest even, saturating.  The gfx950 converter rounds to nearest even but
// turns magnitudes past the last rounding interval into NaN, so values are
// clamped to +-448 first; NaN stays NaN.
__device__ __forceinline__ uint8_t to_e4m3(float x) {
  if (fabsf(x) > 448.0f) x = copysignf(448.0f, x);
  int packed = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false);
  return (uint8_t)(packed & 0xff);
}

__global__ __launch_bounds__(64) void prologue_kernel(StepArgs a) {
  const int t = blockIdx.x;
  const int d = threadIdx.x;
  const int b = t / a.L;
  const int p_in = a.positions[t];
  const int p = p_in < 0 ? 0 : (p_in > a.max_seq_len - 1 ? a.max_seq_len - 1 : p_in);
  const uint16_t *row = a.qkv + (size_t)t * QKV_W;

  // RoPE factors of lane d: pair i = d mod 32 turns by theta = fp32(p) * inv_i,
  // inv_i = base^(-i/32) rounded to fp32; sin/cos of that fp32 angle are taken
  // in double so that large positions keep full accuracy.
  float c = 1.0f, s = 0.0f;
  if (a.sliding) {
    const int i = d & 31;
    const float inv = (float)pow((double)a.rope_base, -(double)i / 32.0);
    const float th = (float)p_in * inv;
    double sd, cd;
    sincos((double)th, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
  }
  const float sgn = d < 32 ? -1.0f : 1.0f;   // x_i c - x_{i+32} s ; x_{i+32} c + x_i s

  const float wq = a.wq[d], wk = a.wk[d];
  const float inv64 = 1.0f / 64.0f;
  // every load of the token first (one memory round trip), then the math
  float x[HQ + 2 * HKV];
#pragma unroll
  for (int h = 0; h < HQ + 2 * HKV; ++h) x[h] = bf16_bits_to_f32(row[h * D + d]);

#pragma unroll
  for (int h = 0; h < HQ; ++h) {
    const float ms = wave_sum(x[h] * x[h]) * inv64;
    float y = x[h] / sqrtf(ms + a.eps) * wq * a.q_scale;
    if (a.sliding) {
      const float partner = __shfl_xor(y, 32, 64);
      y = y * c + sgn * partner * s;
    }
    a.qbuf[((size_t)t * HQ + h) * D + d] = y;
  }

  const uint32_t r = cache_row(a, b, p);
  uint8_t *krow = a.k_cache + (uint64_t)r * ROW;
  uint8_t *vrow = a.v_cache + (uint64_t)r * ROW;
#pragma unroll
  for (int g = 0; g < HKV; ++g) {
    const float xk = x[HQ + g];
    const float ms = wave_sum(xk * xk) * inv64;
    float y = xk / sqrtf(ms + a.eps) * wk;
    if (a.sliding) {
      const float partner = __shfl_xor(y, 32, 64);
      y = y * c + sgn * partner * s;
    }
    krow[g * D + d] = to_e4m3(y / a.kv_scale);
    vrow[g * D + d] = to_e4m3(x[HQ + HKV + g] / a.kv_scale);
  }
}

void launch_prologue(const StepArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(prologue_kernel, dim3(a.B * a.L), dim3(64), 0, stream, a);
}

}  // namespace museattn
