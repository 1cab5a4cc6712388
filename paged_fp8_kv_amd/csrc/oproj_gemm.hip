// The output projection for many tokens as an LDS-tiled bf16 GEMM on gfx950
// MFMA (task page "Whole decoder layer", section "What to compute": the gated
// attention output times o^T; on one GPU the all-reduce after it is the
// identity): y[t][n] = sum_k a[t][k] o[n][k], k < 1024, fp32 sums, bf16 y.
//
// Both operands are K-contiguous rows (a: [T][1024], o: [N][1024]), so one
// MFMA operand fragment is 16 contiguous bytes of a row.  Work-group tile: BM
// rows of o (output features) x BN tokens; its waves form a WAVES_M x WAVES_N
// grid, each wave a block of 16 x 16 tiles on v_mfma_f32_16x16x32_bf16:
//  * A operand = 16 rows of o: lane (n = lane%16, j = lane/16) holds
//    o[row n][k + 8j .. +7]; B operand = 16 tokens of a, the same way; the
//    D tile leaves y[token n][feature 4j .. 4j+3] in lane (n, j) (one 8-byte
//    store);
//  * K moves in stages of 32 through a ring of four LDS stages, filled by the
//    gfx950 direct global -> LDS loads (global_load_lds_dwordx4: each lane's
//    16 bytes land at LDS base + 16 * lane), so three stages are in flight
//    while the waves multiply the fourth, without staging registers.  A
//    stage holds 64-byte rows; the 16-byte slot s of row r holds K-chunk
//    s ^ ((r / 2) % 4), so the 8 lanes of one ds_read_b128 pass (8
//    consecutive rows, one chunk) hit distinct banks.  Each ring stage is its
//    own __shared__ array and the K loop is unrolled by four, so the compiler
//    sees which stage every load and LDS read touches and adds no waits of
//    its own; one barrier per stage;
//  * work-group b takes feature tile b % tiles_m and token tile
//    b / tiles_m: the 8 XCDs take work-groups round-robin, so each XCD's L2
//    holds a few feature tiles of o against a few token tiles at a time.
// No workspace, no state: the launch shape depends on (T, N) only.
#include "device_common.h"
#include "launch.h"

namespace museattn {

namespace {
constexpr int GK = HQ * D;      // 1024: the contraction length
constexpr int BK = 32;          // K per stage: one 16x16x32 K-step
constexpr int RB = BK * 2;      // 64 bytes per staged row

// Stage hand-over: every wave first waits for its own loads of the stage
// (WAIT_VM: vmcnt only, gfx9 encoding with expcnt and lgkmcnt at their
// maxima), then all meet at s_barrier.  No fence: a workgroup-scope fence
// would also wait for the later stages' loads still in flight.  The memory
// clobber keeps the compiler from moving LDS reads across the barrier.
#define LDS_BARRIER() asm volatile("s_barrier" ::: "memory")
#define WAIT_VM(v) \
  __builtin_amdgcn_s_waitcnt(((v) & 0xF) | (0x7 << 4) | (0xF << 8) | (((v) >> 4) << 14))

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Cfg {
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int NQ = (BM + BN) / (16 * NW);   // 16-row load instructions per wave and stage
  static_assert((BM + BN) % (16 * NW) == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
  static constexpr int STAGE = (BM + BN) * RB;
};

template <class C>
__device__ __forceinline__ void issue(uint8_t *base, const uint16_t *const (&src)[C::NQ], int kt,
                                      int wave) {
#pragma unroll
  for (int q = 0; q < C::NQ; ++q)
    __builtin_amdgcn_global_load_lds((const void *)(src[q] + kt * BK),
                                     (__attribute__((address_space(3))) void *)(base + (C::NW * q + wave) * 1024),
                                     16, 0, 0);
}

template <class C>
__device__ __forceinline__ void compute(const uint8_t *base, uint32_t rd_a, uint32_t rd_b,
                                        f32x4 (&acc)[C::TM][C::TN]) {
  bf16x8 af[C::TM], bfr[C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) af[i] = *reinterpret_cast<const bf16x8 *>(base + rd_a + 16 * i * RB);
#pragma unroll
  for (int q = 0; q < C::TN; ++q) bfr[q] = *reinterpret_cast<const bf16x8 *>(base + rd_b + 16 * q * RB);
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int q = 0; q < C::TN; ++q)
      acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[q], acc[i][q], 0, 0, 0);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(const uint16_t *__restrict__ a,
                                             const uint16_t *__restrict__ o,
                                             uint16_t *__restrict__ y, int T, int N, int tiles_m) {
  using C = Cfg<BM, BN, WAVES_M, WAVES_N>;
  constexpr int NK = GK / BK;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[C::STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * BM, t0 = tn * BN;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  const uint16_t *src[C::NQ];
#pragma unroll
  for (int q = 0; q < C::NQ; ++q) {
    const int row = 16 * (C::NW * q + wave) + (lane >> 2);
    const int c = (lane & 3) ^ ((lane >> 3) & 3);
    const uint16_t *p;
    if (row < BM) {
      int r = m0 + row;
      r = r < N ? r : N - 1;
      p = o + (size_t)r * GK;
    } else {
      int r = t0 + row - BM;
      r = r < T ? r : T - 1;
      p = a + (size_t)r * GK;
    }
    src[q] = p + 8 * c;
  }

  f32x4 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int q = 0; q < C::TN; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int slot = 16 * (j ^ ((n >> 1) & 3));
  const uint32_t rd_a = (wm * C::WM + n) * RB + slot;
  const uint32_t rd_b = (BM + wn * C::WN + n) * RB + slot;

  issue<C>(st0, src, 0, wave);
  issue<C>(st1, src, 1, wave);
  issue<C>(st2, src, 2, wave);
#pragma unroll 1
  for (int k0 = 0; k0 < NK - 4; k0 += 4) {
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st3, src, k0 + 3, wave); compute<C>(st0, rd_a, rd_b, acc);
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st0, src, k0 + 4, wave); compute<C>(st1, rd_a, rd_b, acc);
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st1, src, k0 + 5, wave); compute<C>(st2, rd_a, rd_b, acc);
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st2, src, k0 + 6, wave); compute<C>(st3, rd_a, rd_b, acc);
  }
  // the last four stages (NK-4 .. NK-2 already in flight)
  WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st3, src, NK - 1, wave); compute<C>(st0, rd_a, rd_b, acc);
  WAIT_VM(2 * C::NQ); LDS_BARRIER(); compute<C>(st1, rd_a, rd_b, acc);
  WAIT_VM(1 * C::NQ); LDS_BARRIER(); compute<C>(st2, rd_a, rd_b, acc);
  WAIT_VM(0); LDS_BARRIER(); compute<C>(st3, rd_a, rd_b, acc);

#pragma unroll
  for (int q = 0; q < C::TN; ++q) {
    const int t = t0 + wn * C::WN + 16 * q + n;
    if (t >= T) continue;
    uint16_t *yrow = y + (size_t)t * N;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int f = m0 + wm * C::WM + 16 * i + 4 * j;
      if (f >= N) continue;
      const f32x4 v = acc[i][q];
      const uint32_t lo = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<uint2 *>(yrow + f) = uint2{lo, hi};
    }
  }
}
template <int BM, int BN, int WAVES_M, int WAVES_N>
void launch_gemm(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                 hipStream_t stream) {
  const int tiles_m = (N + BM - 1) / BM, tiles_n = (T + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WAVES_M, WAVES_N>), dim3(tiles_m * tiles_n),
                     dim3(64 * WAVES_M * WAVES_N), 0, stream, a, o, y, T, N, tiles_m);
}

int64_t tiles(int T, int N, int bm, int bn) {
  return (int64_t)((N + bm - 1) / bm) * ((T + bn - 1) / bn);
}

}  // namespace

// 256 x 256 tiles (8 waves of 128 x 64, 128 KB of LDS, one work-group per
// CU) once they give every one of the chip's 256 CUs a tile; otherwise
// 128 x 128 (4 waves of 64 x 64, 64 KB, two work-groups per CU).
void gemm_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                hipStream_t stream) {
  if (tiles(T, N, 256, 256) >= 256)
    launch_gemm<256, 256, 2, 4>(a, o, y, T, N, stream);
  else
    launch_gemm<128, 128, 2, 2>(a, o, y, T, N, stream);
}

}  // namespace museattn
