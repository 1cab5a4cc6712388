// The attention output projection that follows the step in the decoder layer
// (task page "Whole decoder layer", section "What to compute": the gated
// attention output times o^T; on one GPU the all-reduce after it is the
// identity): y[t][n] = sum_k a[t][k] o[n][k], a = the step's bf16 output
// [T][1024] (16 heads x 64), o bf16 [N][1024], fp32 accumulation, bf16 y.
//
// Y^T = O . A^T on v_mfma_f32_16x16x32_bf16: the A operand is 16 rows of o
// (lane (n, j) holds o[n0 + n][k + 8j..+7], 16 contiguous bytes), the B
// operand 16 tokens of a (lane (t, j) holds a[t0 + t][k + 8j..+7]), so both
// come straight from row-major memory; the D tile leaves y[t][n0 + 4j..+3] in
// lane (t, j), one 8-byte store.
//
// Work-group (nb, tb): o rows 64nb..64nb+63 (4 tiles of 16), tokens
// 16tb..16tb+15.  Its 4 waves split the 1024-long sum in quarters; each lane
// issues all of its loads at once (8 of a, 32 of o: a decode step's 16 MB of
// o is read in one round trip), a is read once per 64 rows of o, and LDS adds
// the four partial tiles.  Bound: HBM on o for small T.
#include "device_common.h"
#include "launch.h"

namespace museattn {

constexpr int OPROJ_K = HQ * D;   // 1024

__global__ __launch_bounds__(256) void oproj_kernel(const uint16_t *__restrict__ a,
                                                   const uint16_t *__restrict__ o,
                                                   uint16_t *__restrict__ y, int T, int N) {
  __shared__ f32x4 red[4][4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int n0 = blockIdx.x * 64, t0 = blockIdx.y * 16;
  const int kq = wave * (OPROJ_K / 4) + 8 * j;   // this lane's first k
  bf16x8 w[4][8], b[8];
  int t = t0 + n;
  t = t < T ? t : T - 1;   // rows past T are read (valid) and never stored
  const uint16_t *arow = a + (size_t)t * OPROJ_K + kq;
#pragma unroll
  for (int s = 0; s < 8; ++s) b[s] = *reinterpret_cast<const bf16x8 *>(arow + 32 * s);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint16_t *orow = o + (size_t)(n0 + 16 * r + n) * OPROJ_K + kq;
#pragma unroll
    for (int s = 0; s < 8; ++s) w[r][s] = *reinterpret_cast<const bf16x8 *>(orow + 32 * s);
  }
  __builtin_amdgcn_sched_barrier(0);   // all 40 loads in flight before the first product
  f32x4 acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[r][s], b[s], acc[r], 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  // wave r finishes row tile r: lane (t, j) holds y[t0 + t][n0 + 16r + 4j..+3]
  const int r = wave;
  const f32x4 v = red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane];
  if (t0 + n < T) {
    const uint32_t lo = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<uint2 *>(y + (size_t)(t0 + n) * N + n0 + 16 * r + 4 * j) = uint2{lo, hi};
  }
}

void launch_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                  hipStream_t stream) {
  hipLaunchKernelGGL(oproj_kernel, dim3(N / 64, (T + 15) / 16), dim3(256), 0, stream, a, o, y, T, N);
}

}  // namespace museattn
