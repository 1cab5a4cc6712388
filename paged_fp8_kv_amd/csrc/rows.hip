// The new cache rows of a prefill block (L > 8), written before the attention
// kernel reads them (task page "Gated attention decode", section "What to
// compute", the cache line of the listing): for every block token t at
// position p, k = rmsnorm(k) * w_k, rotated on sliding layers, then
// fp8(k / kv_scale) and fp8(v / kv_scale) into cache row row(b, p).  With
// more than 8 block tokens a token's row is read by work-groups that handle
// other tokens, so the rows go in first and the kernel boundary publishes
// them.  (Up to 8 block tokens the attention kernel writes them itself.)
//
// One wave per block token, four tokens per 256-thread work-group; lane =
// dim, each lane normalises, rotates and encodes both KV heads' k and v at
// its dim.  The math is the attention kernel's own.
#include "device_common.h"
#include "launch.h"

namespace museattn {

__global__ __launch_bounds__(256) void rows_kernel(StepArgs a) {
  const int wave = threadIdx.x >> 6, d = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.B * a.L) return;   // uniform over the wave; no barriers below
  const int b = t / a.L;
  int p = a.positions[t];
  p = p < 0 ? 0 : (p > a.max_seq_len - 1 ? a.max_seq_len - 1 : p);
  const uint16_t *row = a.qkv + (size_t)t * QKV_W;
  float k[2], v[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    k[g] = bf16_bits_to_f32(row[K_OFF + g * D + d]);
    v[g] = bf16_bits_to_f32(row[V_OFF + g * D + d]);
  }
  const float wk = a.wk[d];
  const uint64_t base = (uint64_t)cache_row(a, b, p) * ROW + d;
  float2 c = make_float2(1.0f, 0.0f);
  if (a.sliding) c = rope_cs(p, d & 31);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float ms = wave_sum(k[g] * k[g]) * (1.0f / 64.0f);
    float y = k[g] / sqrtf(ms + a.eps) * wk;
    if (a.sliding) {
      const int yi = __float_as_int(y);
      const auto sw = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
      const float partner = __int_as_float(d < 32 ? sw[1] : sw[0]);
      y = d < 32 ? y * c.x - partner * c.y : y * c.x + partner * c.y;
    }
    a.k_cache[base + g * D] = to_e4m3(y / a.kv_scale);
    a.v_cache[base + g * D] = to_e4m3(v[g] / a.kv_scale);
  }
}

void launch_rows(const StepArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(rows_kernel, dim3((a.B * a.L + 3) / 4), dim3(256), 0, stream, a);
}

}  // namespace museattn
