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
//  * K moves in stages of BK (32 or 64) through a ring of four LDS stages,
//    filled by the gfx950 direct global -> LDS loads (global_load_lds_dwordx4:
//    each lane's 16 bytes land at LDS base + 16 * lane), so three stages are
//    in flight while the waves multiply the fourth, without staging
//    registers.  A stage holds rows of 2 BK bytes (4 or 8 chunks of 16 B);
//    chunk c of row r sits at slot c ^ ((r / 2) % chunks), so each 16-lane
//    pass of a ds_read_b128 (gfx950 serves lanes {0-3, 12-15, 20-23, 24-27},
//    {4-7, 8-11, 16-19, 28-31} and the same + 32 together) meets 16 distinct
//    16-byte bank groups.  Each ring stage is its own __shared__ array and the
//    K loop is unrolled by four, so the compiler sees which stage every load
//    and LDS read touches and adds no waits of its own; one barrier per
//    stage.  64-element stages (whole 128-byte lines, 16 stages) serve the
//    4-wave tiles: their K loop is bound by how many bytes a work-group has
//    in flight, and 32-element stages left it at about 16 us whatever the
//    tile;
//  * work-group b takes feature tile b % tiles_m and token tile
//    b / tiles_m: the 8 XCDs take work-groups round-robin, so each XCD's L2
//    holds a few feature tiles of o against a few token tiles at a time.
// No workspace, no state: the launch shape depends on (T, N) only.
#include "device_common.h"
#include "launch.h"

namespace museattn {

namespace {
constexpr int GK = HQ * D;      // 1024: the contraction length

// Stage hand-over: every wave first waits for its own loads of the stage
// (WAIT_VM: vmcnt only, gfx9 encoding with expcnt and lgkmcnt at their
// maxima), then all meet at s_barrier.  No fence: a workgroup-scope fence
// would also wait for the later stages' loads still in flight.  The memory
// clobber keeps the compiler from moving LDS reads across the barrier.
#define LDS_BARRIER() asm volatile("s_barrier" ::: "memory")
#define WAIT_VM(v) \
  __builtin_amdgcn_s_waitcnt(((v) & 0xF) | (0x7 << 4) | (0xF << 8) | (((v) >> 4) << 14))

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK_>
struct Cfg {
  static constexpr int BK = BK_;             // K per stage (32 or 64)
  static constexpr int RB = 2 * BK;          // bytes of one staged row
  static constexpr int CPR = RB / 16;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;       // rows one load instruction fills
  static constexpr int KS = BK / 32;         // 16x16x32 K-steps per stage
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int NQ = (BM + BN) / (RPI * NW);   // load instructions per wave and stage
  static_assert((BK == 32 || BK == 64) && (BM + BN) % (RPI * NW) == 0 && WM % 16 == 0 &&
                    WN % 16 == 0, "tile shape");
  static constexpr int STAGE = (BM + BN) * RB;
};

template <class C>
__device__ __forceinline__ void issue(uint8_t *base, const uint16_t *const (&src)[C::NQ], int kt,
                                      int wave) {
#pragma unroll
  for (int q = 0; q < C::NQ; ++q)
    __builtin_amdgcn_global_load_lds((const void *)(src[q] + kt * C::BK),
                                     (__attribute__((address_space(3))) void *)(base + (C::NW * q + wave) * 1024),
                                     16, 0, 0);
}

// One stage's products: K-step ks reads chunk 4 ks + j of each of the
// wave's rows (lane (n, j)); rd_a, rd_b: the lane's row offsets.
template <class C>
__device__ __forceinline__ void compute(const uint8_t *base, uint32_t rd_a, uint32_t rd_b, int n,
                                        int j, f32x4 (&acc)[C::TM][C::TN]) {
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t slot = 16 * ((4 * ks + j) ^ ((n >> 1) & (C::CPR - 1)));
    bf16x8 af[C::TM], bfr[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      af[i] = *reinterpret_cast<const bf16x8 *>(base + rd_a + slot + 16 * i * C::RB);
#pragma unroll
    for (int q = 0; q < C::TN; ++q)
      bfr[q] = *reinterpret_cast<const bf16x8 *>(base + rd_b + slot + 16 * q * C::RB);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int q = 0; q < C::TN; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[q], acc[i][q], 0, 0, 0);
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(const uint16_t *__restrict__ a,
                                             const uint16_t *__restrict__ o,
                                             uint16_t *__restrict__ y, int T, int N, int tiles_m) {
  using C = Cfg<BM, BN, WAVES_M, WAVES_N, BK>;
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
    const int row = C::RPI * (C::NW * q + wave) + lane / C::CPR;
    const int c = (lane % C::CPR) ^ ((row >> 1) & (C::CPR - 1));
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

  const uint32_t rd_a = (wm * C::WM + n) * C::RB;
  const uint32_t rd_b = (BM + wn * C::WN + n) * C::RB;

  issue<C>(st0, src, 0, wave);
  issue<C>(st1, src, 1, wave);
  issue<C>(st2, src, 2, wave);
#pragma unroll 1
  for (int k0 = 0; k0 < NK - 4; k0 += 4) {
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st3, src, k0 + 3, wave); compute<C>(st0, rd_a, rd_b, n, j, acc);
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st0, src, k0 + 4, wave); compute<C>(st1, rd_a, rd_b, n, j, acc);
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st1, src, k0 + 5, wave); compute<C>(st2, rd_a, rd_b, n, j, acc);
    WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st2, src, k0 + 6, wave); compute<C>(st3, rd_a, rd_b, n, j, acc);
  }
  // the last four stages (NK-4 .. NK-2 already in flight)
  WAIT_VM(2 * C::NQ); LDS_BARRIER(); issue<C>(st3, src, NK - 1, wave); compute<C>(st0, rd_a, rd_b, n, j, acc);
  WAIT_VM(2 * C::NQ); LDS_BARRIER(); compute<C>(st1, rd_a, rd_b, n, j, acc);
  WAIT_VM(1 * C::NQ); LDS_BARRIER(); compute<C>(st2, rd_a, rd_b, n, j, acc);
  WAIT_VM(0); LDS_BARRIER(); compute<C>(st3, rd_a, rd_b, n, j, acc);

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
template <int BM, int BN, int WAVES_M, int WAVES_N, int BK>
void launch_gemm(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                 hipStream_t stream) {
  const int tiles_m = (N + BM - 1) / BM, tiles_n = (T + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WAVES_M, WAVES_N, BK>), dim3(tiles_m * tiles_n),
                     dim3(64 * WAVES_M * WAVES_N), 0, stream, a, o, y, T, N, tiles_m);
}

int64_t tiles(int T, int N, int bm, int bn) {
  return (int64_t)((N + bm - 1) / bm) * ((T + bn - 1) / bn);
}

}  // namespace

#ifndef MUSEATTN_GEMM_CFG
#define MUSEATTN_GEMM_CFG 0   // 0: chosen by shape; 1-5 force one tile shape
#endif

// Tile shapes (feature rows of o x tokens, waves):
//   1: 256 x 256, 8 waves of 128 x 64, 32-element stages (128 KB of LDS)
//   2: 128 x 128, 4 waves of 64 x 64, 64-element stages (128 KB)
//   3: 128 x 64, 4 waves of 64 x 32, 64-element stages (96 KB)
//   4: 128 x 192, 8 waves of 64 x 48, 64-element stages (160 KB)
//   5: 256 x 128, 8 waves of 64 x 64, 32-element stages (96 KB)
// Every shape takes one work-group per CU (LDS), so a launch runs in
// ceil(tiles / 256) rounds on the chip's 256 CUs.  The shape with the least
// estimated time wins, from the measured time of its first full round of
// tiles and of each further round (hidden 8192; later rounds overlap the
// previous round's tail): a partly filled round costs as much as a full one.
static int gemm_cfg(int T, int N) {
  if (MUSEATTN_GEMM_CFG) return MUSEATTN_GEMM_CFG;
  struct Shape { int id, bm, bn; float first_us, next_us; };
  static constexpr Shape shapes[] = {{3, 128, 64, 12.f, 11.f}, {2, 128, 128, 16.5f, 14.f},
                                     {4, 128, 192, 19.f, 15.5f}, {5, 256, 128, 25.5f, 21.f},
                                     {1, 256, 256, 41.f, 40.f}};
  int best = 1;
  float best_t = 0.f;
  for (const Shape &sh : shapes) {
    const int64_t rounds = (tiles(T, N, sh.bm, sh.bn) + 255) / 256;
    const float t = sh.first_us + (float)(rounds - 1) * sh.next_us;
    if (best_t == 0.f || t < best_t) {
      best = sh.id;
      best_t = t;
    }
  }
  return best;
}

void gemm_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N,
                hipStream_t stream) {
  switch (gemm_cfg(T, N)) {
    case 1: launch_gemm<256, 256, 2, 4, 32>(a, o, y, T, N, stream); break;
    case 5: launch_gemm<256, 128, 4, 2, 32>(a, o, y, T, N, stream); break;
    case 4: launch_gemm<128, 192, 2, 4, 64>(a, o, y, T, N, stream); break;
    case 2: launch_gemm<128, 128, 2, 2, 64>(a, o, y, T, N, stream); break;
    default: launch_gemm<128, 64, 2, 2, 64>(a, o, y, T, N, stream); break;
  }
}

}  // namespace museattn
