// A memory-system probe, not part of the step: the read rate of the step's
// own K/V row gather.  It reads every visible key's K and V rows of a
// full-layer decode step (positions 0 .. seq_lens[b] - 1 of each request,
// through the page table) with the attention kernel's decode loads and
// concurrency -- 256 work-groups of 8 waves, each taking an equal share of
// all requests' 32-key chunks, the row ids of up to 4096 keys staged in LDS,
// the same load instructions per chunk, two chunks in flight per wave -- and
// folds the bytes into one checksum per work-group, so no load can be
// dropped.  Its time is the ceiling the attention kernel would reach if its
// arithmetic were free.
#include "device_common.h"
#include "launch.h"

namespace museattn {

namespace {

constexpr int PROBE_ROWS_LDS = 4096;   // row ids staged per piece

struct ProbeRows {
  uint4 k[4];   // 16-byte pieces of the K rows of keys n and 16 + n
  uint2 v[8];   // 8-byte pieces of the V rows of the 8 keys 4j.. and 16 + 4j..
};

// The attention kernel's own decode loads of one 32-key chunk (8 KB): lane
// (n = lane%16, j = lane/16) reads bytes 16j .. and 64 + 16j .. of the K rows
// of keys n and 16 + n, and bytes 8n .. 8n + 7 of the V rows of keys 4j ..
// 4j + 3 and 16 + 4j .. 16 + 4j + 3 (one V load instruction covers 4 whole
// rows).
__device__ __forceinline__ void probe_load(ProbeRows &r, const uint8_t *__restrict__ kc,
                                           const uint8_t *__restrict__ vc, const uint32_t *rows,
                                           int n, int j) {
  const uint64_t r0 = rows[n], r1 = rows[16 + n];
  const uint8_t *k0 = kc + r0 * ROW + 16 * j, *k1 = kc + r1 * ROW + 16 * j;
  r.k[0] = *reinterpret_cast<const uint4 *>(k0);
  r.k[1] = *reinterpret_cast<const uint4 *>(k0 + 64);
  r.k[2] = *reinterpret_cast<const uint4 *>(k1);
  r.k[3] = *reinterpret_cast<const uint4 *>(k1 + 64);
  const uint4 va = *reinterpret_cast<const uint4 *>(rows + 4 * j);
  const uint4 vb = *reinterpret_cast<const uint4 *>(rows + 16 + 4 * j);
  const uint32_t vr[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r.v[i] = *reinterpret_cast<const uint2 *>(vc + (uint64_t)vr[i] * ROW + 8 * n);
}

__device__ __forceinline__ uint32_t probe_fold(const ProbeRows &r) {
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) x ^= r.k[i].x ^ r.k[i].y ^ r.k[i].z ^ r.k[i].w;
#pragma unroll
  for (int i = 0; i < 8; ++i) x ^= r.v[i].x ^ r.v[i].y;
  return x;
}

__global__ __launch_bounds__(THREADS) void gather_probe_kernel(
    const int32_t *__restrict__ table, const int32_t *__restrict__ seq_lens,
    const uint8_t *__restrict__ kc, const uint8_t *__restrict__ vc, int B, int table_stride,
    int max_seq_len, int page_size, int64_t num_rows, uint32_t *__restrict__ out) {
  __shared__ int pref[MAX_BATCH + 1];
  __shared__ int scan[WAVES];
  __shared__ uint32_t rows[PROBE_ROWS_LDS];
  __shared__ uint32_t red[WAVES];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const int shift = page_size == 1 ? 0 : 6;
  const uint32_t units = (uint32_t)(num_rows >> shift);

  // chunk counts of the requests (two per thread) and their prefix sums
  int cnt[2], sl[2], sum = 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int b = 2 * tid + k;
    sl[k] = b < B ? seq_lens[b] : 0;
    sl[k] = sl[k] < 0 ? 0 : (sl[k] > max_seq_len ? max_seq_len : sl[k]);
    cnt[k] = (sl[k] + CHUNK - 1) / CHUNK;
    sum += cnt[k];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    incl += lane >= off ? v : 0;
  }
  if (lane == 63) scan[wave] = incl;
  __syncthreads();
  int run = incl - sum;
#pragma unroll
  for (int w2 = 0; w2 < WAVES; ++w2) run += w2 < wave ? scan[w2] : 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (2 * tid + k < B) pref[2 * tid + k] = run;
    run += cnt[k];
  }
  if (tid == 0) {
    int total = 0;
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2) total += scan[w2];
    pref[B] = total;
  }
  __syncthreads();

  const int64_t C = pref[B];
  const int G = gridDim.x;
  const int64_t cb = div_floor((int64_t)blockIdx.x * C, G);
  const int64_t ce = div_floor((int64_t)(blockIdx.x + 1) * C, G);
  uint32_t acc = 0;
  int b = 0;
  while (b < B - 1 && pref[b + 1] <= cb) ++b;
  for (; b < B && pref[b] < ce; ++b) {
    const int x = (int)((cb > pref[b] ? cb : pref[b]) - pref[b]);
    const int y = (int)((ce < pref[b + 1] ? ce : pref[b + 1]) - pref[b]);
    const int len = seq_lens[b] < 0 ? 0 : (seq_lens[b] > max_seq_len ? max_seq_len : seq_lens[b]);
    for (int p0 = x; p0 < y; p0 += PROBE_ROWS_LDS / CHUNK) {   // pieces of 4096 keys
      const int p1 = p0 + PROBE_ROWS_LDS / CHUNK < y ? p0 + PROBE_ROWS_LDS / CHUNK : y;
      __syncthreads();   // the previous piece's row ids are no longer read
      for (int i = tid; i < PROBE_ROWS_LDS; i += THREADS) {
        int u = p0 * CHUNK + i;
        u = u < len - 1 ? u : len - 1;   // keys past the request repeat its last row
        uint32_t un = (uint32_t)table[(int64_t)b * table_stride + (u >> shift)];
        un = un < units ? un : units - 1;
        rows[i] = (un << shift) + (uint32_t)(u & (page_size - 1));
      }
      __syncthreads();
      // this wave's chunks of the piece: wave, wave + 8, ... with two in flight
      const int nch = p1 - p0;
      const int nloc = nch > wave ? (nch - wave + WAVES - 1) / WAVES : 0;
      if (nloc > 0) {
        const int last = nloc - 1;
        auto rows_of = [&](int i) { return rows + (wave + (i < last ? i : last) * WAVES) * CHUNK; };
        ProbeRows r0, r1;
        probe_load(r0, kc, vc, rows_of(0), n, j);
        probe_load(r1, kc, vc, rows_of(1), n, j);
        int i = 0;
        for (; i + 2 <= nloc; i += 2) {
          acc ^= probe_fold(r0);
          probe_load(r0, kc, vc, rows_of(i + 2), n, j);
          acc ^= probe_fold(r1);
          probe_load(r1, kc, vc, rows_of(i + 3), n, j);
        }
        if (i < nloc) acc ^= probe_fold(r0);
      }
    }
  }
  // one checksum per work-group
  acc ^= __shfl_xor(acc, 32);
  acc ^= __shfl_xor(acc, 16);
  acc ^= __shfl_xor(acc, 8);
  acc ^= __shfl_xor(acc, 4);
  acc ^= __shfl_xor(acc, 2);
  acc ^= __shfl_xor(acc, 1);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2) x ^= red[w2];
    out[blockIdx.x] = x;
  }
}

}  // namespace

void launch_gather_probe(const int32_t *table, const int32_t *seq_lens, const uint8_t *kc,
                         const uint8_t *vc, int B, int table_stride, int max_seq_len,
                         int page_size, int64_t num_rows, uint32_t *out, int work_groups,
                         hipStream_t stream) {
  hipLaunchKernelGGL(gather_probe_kernel, dim3(work_groups), dim3(THREADS), 0, stream, table,
                     seq_lens, kc, vc, B, table_stride, max_seq_len, page_size, num_rows, out);
}

}  // namespace museattn
