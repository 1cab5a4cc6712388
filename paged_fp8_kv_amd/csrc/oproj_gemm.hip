// The output projection for many tokens as an LDS-tiled bf16 GEMM on gfx950
// MFMA (task page "Whole decoder layer", section "What to compute": the gated
// attention output times o^T; on one GPU the all-reduce after it is the
// identity): y[t][n] = sum_k a[t][k] o[n][k], k < 1024, fp32 sums, bf16 y.
//
// Both operands are K-contiguous rows (a: [T][1024], o: [N][1024]), so one
// MFMA operand fragment is 16 contiguous bytes of a row.  Work-group tile: BM
// rows of o (output features) x BN tokens, 4 waves in a 2 x 2 grid, each wave
// a (BM/2) x (BN/2) block of 16 x 16 tiles on v_mfma_f32_16x16x32_bf16:
//  * A operand = 16 rows of o: lane (n = lane%16, j = lane/16) holds
//    o[row n][k + 8j .. +7]; B operand = 16 tokens of a, the same way; the
//    D tile leaves y[token n][feature 4j .. 4j+3] in lane (n, j) (one 8-byte
//    store);
//  * K moves in stages of 64: each thread loads 16-byte pieces of the next
//    stage's rows into registers while the waves multiply the current stage
//    out of LDS; rows sit in LDS at a 144-byte stride (128 + 16), so the 8
//    lanes of one ds_read_b128 / ds_write_b128 pass hit distinct banks;
//    two LDS buffers, one barrier per stage;
//  * work-group b takes feature tile b % tiles_m and token tile
//    b / tiles_m: the 8 XCDs take work-groups round-robin, so each XCD's L2
//    holds a quarter of o's rows against a few token tiles at a time.
// No workspace, no state: the launch shape depends on (T, N) only.
#include "device_common.h"
#include "launch.h"

namespace museattn {

namespace {

constexpr int GK = HQ * D;     // 1024: the contraction length
constexpr int GBK = 64;        // K per stage
constexpr int GRS = GBK * 2 + 16;   // LDS bytes per staged row (padded)
// staged pieces as native vectors: arrays of HIP's uint4 (a union type) were
// kept in memory (spare LDS or scratch) instead of registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int BM, int BN>
struct GemmLds {
  uint8_t buf[2][(BM + BN) * GRS];
};

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ a,
                                                  const uint16_t *__restrict__ o,
                                                  uint16_t *__restrict__ y, int T, int N,
                                                  int tiles_m) {
  constexpr int WM = BM / 2, WN = BN / 2;      // wave block
  constexpr int TM = WM / 16, TN = WN / 16;    // 16 x 16 tiles per wave
  constexpr int LA = BM * 8 / 256, LB = BN * 8 / 256;   // 16-byte pieces per thread and stage
  static_assert(BM % 32 == 0 && BN % 32 == 0 && LA >= 1 && LB >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) GemmLds<BM, BN> sh;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * BM, t0 = tn * BN;
  const int wm = wave & 1, wn = wave >> 1;

  // this thread's staged pieces: row tid/8 + 32i, piece tid%8 of the stage
  // (rows past N or T are read clamped and never stored)
  const int prow = tid >> 3, pcol = tid & 7;
  const uint16_t *ga = o + (size_t)(m0 + prow) * GK + pcol * 8;
  const uint16_t *gb = a + (size_t)(t0 + prow) * GK + pcol * 8;
  int ra_off[LA], rb_off[LB];   // element offsets of rows 32i from the first
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = m0 + prow + 32 * i;
    ra_off[i] = ((r < N ? r : N - 1) - (m0 + prow)) * GK;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = t0 + prow + 32 * i;
    rb_off[i] = ((r < T ? r : T - 1) - (t0 + prow)) * GK;
  }
  const uint32_t st_off = prow * GRS + pcol * 16;   // LDS byte offset of row prow

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int q = 0; q < TN; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NK = GK / GBK;
  u32x4 ra[LA], rb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4 *>(ga + ra_off[i]);
#pragma unroll
  for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(gb + rb_off[i]);
#pragma unroll
  for (int i = 0; i < LA; ++i)
    *reinterpret_cast<u32x4 *>(sh.buf[0] + st_off + 32 * i * GRS) = ra[i];
#pragma unroll
  for (int i = 0; i < LB; ++i)
    *reinterpret_cast<u32x4 *>(sh.buf[0] + st_off + (BM + 32 * i) * GRS) = rb[i];
  __syncthreads();

  const uint32_t rd_a = (wm * WM + n) * GRS + 16 * j;        // LDS operand reads
  const uint32_t rd_b = (BM + wn * WN + n) * GRS + 16 * j;
#pragma unroll 1
  for (int kt = 0; kt < NK; ++kt) {
    const bool more = kt + 1 < NK;   // uniform
    if (more) {   // the next stage's pieces, in flight during this stage's products
      const int k1 = (kt + 1) * GBK;
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4 *>(ga + ra_off[i] + k1);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(gb + rb_off[i] + k1);
    }
    const uint8_t *base = sh.buf[kt & 1];
#pragma unroll
    for (int kk = 0; kk < GBK / 32; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8 *>(base + rd_a + 16 * i * GRS + 64 * kk);
#pragma unroll
      for (int q = 0; q < TN; ++q)
        bfr[q] = *reinterpret_cast<const bf16x8 *>(base + rd_b + 16 * q * GRS + 64 * kk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < TN; ++q)
          acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[q], acc[i][q], 0, 0, 0);
    }
    if (more) {
      uint8_t *nb = sh.buf[(kt + 1) & 1];
#pragma unroll
      for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4 *>(nb + st_off + 32 * i * GRS) = ra[i];
#pragma unroll
      for (int i = 0; i < LB; ++i)
        *reinterpret_cast<u32x4 *>(nb + st_off + (BM + 32 * i) * GRS) = rb[i];
    }
    __syncthreads();
  }

  // D tile (i, q): rows (features) m0 + wm*WM + 16i + 4j + r, column (token)
  // t0 + wn*WN + 16q + n
#pragma unroll
  for (int q = 0; q < TN; ++q) {
    const int t = t0 + wn * WN + 16 * q + n;
    if (t >= T) continue;
    uint16_t *yrow = y + (size_t)t * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int f = m0 + wm * WM + 16 * i + 4 * j;
      if (f >= N) continue;   // N is a multiple of 64: a 4-feature group is whole
      const f32x4 v = acc[i][q];
      const uint32_t lo = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<uint2 *>(yrow + f) = uint2{lo, hi};
    }
  }
}

template <int BM, int BN>
void launch_gemm(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                 hipStream_t stream) {
  const int tiles_m = (N + BM - 1) / BM, tiles_n = (T + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<BM, BN>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, a, o,
                     y, T, N, tiles_m);
}

int64_t tiles(int T, int N, int bm, int bn) {
  return (int64_t)((N + bm - 1) / bm) * ((T + bn - 1) / bn);
}

}  // namespace

// The largest tile that still gives the chip's 256 CUs about two work-groups
// each (one for the largest tile), so short token counts are not left to a
// few CUs.
void gemm_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                hipStream_t stream) {
  if (tiles(T, N, 256, 128) >= 512)
    launch_gemm<256, 128>(a, o, y, T, N, stream);
  else if (tiles(T, N, 128, 128) >= 256)
    launch_gemm<128, 128>(a, o, y, T, N, stream);
  else
    launch_gemm<128, 64>(a, o, y, T, N, stream);
}

}  // namespace museattn
