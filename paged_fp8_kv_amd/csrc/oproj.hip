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
// Work-group x owns o rows 32x..32x+31 (N/32 work-groups: 256 at N = 8192,
// one per CU) and keeps them in registers while it passes over the tokens 64
// at a time (work-group y takes passes y, y + gridDim.y, ...), so o leaves
// HBM once when T <= 64 and a, which every work-group reads, stays in L2.
// Its 4 waves split the 1024-long sum in quarters; each lane issues all of
// its loads of a pass before the first product, and LDS adds the quarters.
// Bound: HBM on o for small T.
#include "device_common.h"
#include "launch.h"

namespace museattn {

constexpr int OPROJ_K = HQ * D;   // 1024
constexpr int OP_ROWS = 32;       // rows of o per work-group
constexpr int OP_TOK = 64;        // tokens per pass (4 tiles of 16)
constexpr int OP_MAX_PASS_GROUPS = 1024;

// One pass over tokens t0..t0 + 16 NTT - 1 (rows past T are read clamped and
// never stored).
template <int NTT>
__device__ __forceinline__ void oproj_pass(const uint16_t *__restrict__ a,
                                           uint16_t *__restrict__ y, const bf16x8 (&w)[2][8],
                                           f32x4 (&red)[4][2][4][64], int t0, int T, int N,
                                           int n0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int kq = wave * (OPROJ_K / 4) + 8 * j;
  bf16x8 b[NTT][8];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    int t = t0 + 16 * tt + n;
    t = t < T ? t : T - 1;
    const uint16_t *arow = a + (size_t)t * OPROJ_K + kq;
#pragma unroll
    for (int s = 0; s < 8; ++s) b[tt][s] = *reinterpret_cast<const bf16x8 *>(arow + 32 * s);
  }
  __builtin_amdgcn_sched_barrier(0);   // all loads in flight before the first product
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[r][s], b[tt][s], acc, 0, 0, 0);
      red[wave][r][tt][lane] = acc;
    }
  }
  __syncthreads();
  // the 2 x NTT tiles go round the waves: tile (r, tt) = (idx / NTT, idx % NTT)
  for (int idx = wave; idx < 2 * NTT; idx += 4) {
    const int r = idx / NTT, tt = idx % NTT;
    const f32x4 v = red[0][r][tt][lane] + red[1][r][tt][lane] + red[2][r][tt][lane] +
                    red[3][r][tt][lane];
    const int t = t0 + 16 * tt + n;
    if (t < T) {
      const uint32_t lo = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<uint2 *>(y + (size_t)t * N + n0 + 16 * r + 4 * j) = uint2{lo, hi};
    }
  }
  __syncthreads();   // red is free for the next pass
}

__global__ __launch_bounds__(256) void oproj_kernel(const uint16_t *__restrict__ a,
                                                   const uint16_t *__restrict__ o,
                                                   uint16_t *__restrict__ y, int T, int N) {
  __shared__ f32x4 red[4][2][4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int n0 = blockIdx.x * OP_ROWS;
  const int kq = wave * (OPROJ_K / 4) + 8 * j;   // this lane's first k
  bf16x8 w[2][8];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint16_t *orow = o + (size_t)(n0 + 16 * r + n) * OPROJ_K + kq;
#pragma unroll
    for (int s = 0; s < 8; ++s) w[r][s] = *reinterpret_cast<const bf16x8 *>(orow + 32 * s);
  }
  for (int t0 = blockIdx.y * OP_TOK; t0 < T; t0 += gridDim.y * OP_TOK) {
    const int left = T - t0;   // uniform
    if (left > 32) oproj_pass<4>(a, y, w, red, t0, T, N, n0);
    else if (left > 16) oproj_pass<2>(a, y, w, red, t0, T, N, n0);
    else oproj_pass<1>(a, y, w, red, t0, T, N, n0);
  }
}

// From this many tokens on, the LDS-tiled GEMM (oproj_gemm.hip) runs the
// projection: this kernel re-reads a once per 32 rows of o, and its per-lane
// loads keep fewer bytes in flight than the GEMM's direct-to-LDS ring
// (hidden 8192, kernel times: T 32 6.8 vs 8.2 us, 64 8.9 vs 8.5, 128 14.6
// vs 8.8).
#ifndef MUSEATTN_OPROJ_GEMM_MIN_T
#define MUSEATTN_OPROJ_GEMM_MIN_T 64
#endif
constexpr int OP_GEMM_MIN_T = MUSEATTN_OPROJ_GEMM_MIN_T;

void launch_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                  hipStream_t stream) {
  if (T >= OP_GEMM_MIN_T) {
    gemm_oproj(a, o, y, T, N, stream);
    return;
  }
  int passes = (T + OP_TOK - 1) / OP_TOK;
  passes = passes < OP_MAX_PASS_GROUPS ? passes : OP_MAX_PASS_GROUPS;
  hipLaunchKernelGGL(oproj_kernel, dim3(N / OP_ROWS, passes), dim3(256), 0, stream, a, o, y, T, N);
}

}  // namespace museattn
