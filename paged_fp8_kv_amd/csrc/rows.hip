// The new cache rows of a prefill block (L > 8), written before the attention
// kernel reads them (task page "Gated attention decode", section "What to
// compute", the cache line of the listing): for every block token t at
// position p, k = rmsnorm(k) * w_k, rotated on sliding layers, then
// fp8(k / kv_scale) and fp8(v / kv_scale) into cache row row(b, p).  With
// more than 8 block tokens a token's row is read by work-groups that handle
// other tokens, so the rows go in first and the kernel boundary publishes
// them.  (Up to 8 block tokens the attention kernel writes them itself.)
//
// One 256-thread work-group per block token: wave 0/1 take k head 0/1, wave
// 2/3 v head 0/1; lane = dim.  The math is the attention kernel's own.
#include "device_common.h"
#include "launch.h"

namespace museattn {

__global__ __launch_bounds__(256) void rows_kernel(StepArgs a) {
  const int t = blockIdx.x, b = t / a.L;
  const int wave = threadIdx.x >> 6, d = threadIdx.x & 63;
  const bool is_k = wave < 2;
  const int g = wave & 1;
  int p = a.positions[t];
  p = p < 0 ? 0 : (p > a.max_seq_len - 1 ? a.max_seq_len - 1 : p);
  float y = bf16_bits_to_f32(a.qkv[(size_t)t * QKV_W + (is_k ? K_OFF : V_OFF) + g * D + d]);
  if (is_k) {   // uniform over the wave
    const float ms = wave_sum(y * y) * (1.0f / 64.0f);
    y = y / sqrtf(ms + a.eps) * a.wk[d];
    if (a.sliding) {
      const int yi = __float_as_int(y);
      const auto sw = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
      const float partner = __int_as_float(d < 32 ? sw[1] : sw[0]);
      const float2 c = rope_cs(p, d & 31);
      y = d < 32 ? y * c.x - partner * c.y : y * c.x + partner * c.y;
    }
  }
  uint8_t *dst = (is_k ? a.k_cache : a.v_cache) + (uint64_t)cache_row(a, b, p) * ROW + g * D + d;
  *dst = to_e4m3(y / a.kv_scale);
}

void launch_rows(const StepArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(rows_kernel, dim3(a.B * a.L), dim3(256), 0, stream, a);
}

}  // namespace museattn
