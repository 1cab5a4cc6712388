// A memory-system probe, not part of the step: how fast this part can read
// the step's K/V rows with nothing else to do.  It reads both rows of every
// visible key of a full-layer decode step (positions 0 .. seq_lens[b] - 1 of
// each request, through the page table) exactly once and folds their 32-bit
// words into one XOR checksum per work-group, so no load can be dropped.
//
// It is built as the fastest plain gather found on this part, not as a copy
// of the attention kernel's loads, so that its time is the ceiling for the
// step's gather: work-group w takes keys [w K / G, (w + 1) K / G) of the K
// keys of all requests laid end to end; it stages the row ids of up to 12,288
// of them in LDS (all table loads issued before the first store: one round
// trip); each wave then walks its own contiguous share in groups of 16 keys,
// lane l reading bytes 16 (l % 8) .. + 15 of the K and V rows of key l / 8 of
// a batch of 8 (8 lanes cover a 128-byte row), with two groups (8 KB per
// wave) in flight.  The row loads are non-temporal: each row is read once,
// and not filling the caches with it made the gather 7-8% faster on decode B
// 32 (672 MB of rows) and 1-3% at B 16.  Deeper rings, 16-wave or two-per-CU
// work-groups and direct-to-LDS loads measured the same as this layout.
#include "device_common.h"
#include "launch.h"

namespace museattn {

namespace {

constexpr int PROBE_IDS = 12288;              // row ids staged per piece (48 KB)
constexpr int PROBE_PER_THREAD = PROBE_IDS / THREADS;
constexpr int PROBE_BATCHES = 2;              // batches of 8 keys per group
constexpr int PROBE_KPG = 8 * PROBE_BATCHES;  // keys per group
constexpr int PROBE_RING = 2;                 // groups in flight per wave

struct ProbeGroup {
  uint4 k[PROBE_BATCHES], v[PROBE_BATCHES];
};

__global__ __launch_bounds__(THREADS) void gather_probe_kernel(
    const int32_t *__restrict__ table, const int32_t *__restrict__ seq_lens,
    const uint8_t *__restrict__ kc, const uint8_t *__restrict__ vc, int B, int table_stride,
    int max_seq_len, int page_size, int64_t num_rows, uint32_t *__restrict__ out) {
  __shared__ int64_t pref[MAX_BATCH + 1];
  __shared__ int64_t scan[WAVES];
  __shared__ uint32_t sid[PROBE_IDS];
  __shared__ uint32_t red[WAVES];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int shift = page_size == 1 ? 0 : 6;
  const uint32_t units = (uint32_t)(num_rows >> shift);

  // key counts of the requests (two per thread) and their prefix sums
  int64_t sum = 0;
  int sl[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int b = 2 * tid + k;
    sl[k] = b < B ? seq_lens[b] : 0;
    sl[k] = sl[k] < 0 ? 0 : (sl[k] > max_seq_len ? max_seq_len : sl[k]);
    sum += sl[k];
  }
  int64_t incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off);
    incl += lane >= off ? v : 0;
  }
  if (lane == 63) scan[wave] = incl;
  __syncthreads();
  int64_t run = incl - sum;
#pragma unroll
  for (int w2 = 0; w2 < WAVES; ++w2) run += w2 < wave ? scan[w2] : 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (2 * tid + k < B) pref[2 * tid + k] = run;
    run += sl[k];
  }
  if (tid == 0) {
    int64_t total = 0;
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2) total += scan[w2];
    pref[B] = total;
  }
  __syncthreads();

  const int64_t K = pref[B];
  const int G = gridDim.x;
  const int64_t kb = div_floor((int64_t)blockIdx.x * K, G);
  const int64_t ke = div_floor((int64_t)(blockIdx.x + 1) * K, G);
  const int sub = lane >> 3, part = lane & 7;
  uint32_t acc = 0;
  for (int64_t p0 = kb; p0 < ke; p0 += PROBE_IDS) {
    const int cnt = (int)(ke - p0 < PROBE_IDS ? ke - p0 : PROBE_IDS);
    __syncthreads();   // the previous piece's row ids are no longer read
    // this thread's keys p0 + tid + i * THREADS (clamped to the piece): their
    // request by a binary search for the first and a walk for the rest, then
    // every table load, then every store
    int64_t key0 = p0 + (tid < cnt ? tid : cnt - 1);
    int lo = 0, hi = B - 1;   // last request b with pref[b] <= key0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= key0) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    const int32_t *src[PROBE_PER_THREAD];
    int low[PROBE_PER_THREAD];
#pragma unroll
    for (int i = 0; i < PROBE_PER_THREAD; ++i) {
      const int ki = tid + i * THREADS;
      const int64_t key = p0 + (ki < cnt ? ki : cnt - 1);
      while (b < B - 1 && pref[b + 1] <= key) ++b;
      const int u = (int)(key - pref[b]);
      src[i] = table + (int64_t)b * table_stride + (u >> shift);
      low[i] = u & (page_size - 1);
    }
    int32_t ent[PROBE_PER_THREAD];
#pragma unroll
    for (int i = 0; i < PROBE_PER_THREAD; ++i) ent[i] = *src[i];
#pragma unroll
    for (int i = 0; i < PROBE_PER_THREAD; ++i) {
      uint32_t un = (uint32_t)ent[i];
      un = un < units ? un : units - 1;
      const int ki = tid + i * THREADS;
      if (ki < cnt) sid[ki] = (un << shift) + (uint32_t)low[i];
    }
    __syncthreads();

    const int ng = (cnt + PROBE_KPG - 1) / PROBE_KPG;
    const int gb = wave * ng / WAVES;
    const int n = (wave + 1) * ng / WAVES - gb;
    if (n > 0) {
      // loads are unconditional (indices clamped into the share), so the
      // compiler can count them and wait only for the group it folds next
      auto issue = [&](ProbeGroup &grp, int g) {
        const int gg = gb + (g < n ? g : n - 1);
#pragma unroll
        for (int u = 0; u < PROBE_BATCHES; ++u) {
          int key = gg * PROBE_KPG + u * 8 + sub;
          key = key < cnt ? key : cnt - 1;
          const uint64_t r = sid[key];
          grp.k[u] = load_nt16(kc + r * ROW + part * 16);
          grp.v[u] = load_nt16(vc + r * ROW + part * 16);
        }
      };
      auto fold = [&](const ProbeGroup &grp, int g) {
#pragma unroll
        for (int u = 0; u < PROBE_BATCHES; ++u) {
          const int key = (gb + g) * PROBE_KPG + u * 8 + sub;
          const uint32_t x = grp.k[u].x ^ grp.k[u].y ^ grp.k[u].z ^ grp.k[u].w ^ grp.v[u].x ^
                             grp.v[u].y ^ grp.v[u].z ^ grp.v[u].w;
          acc ^= key < cnt ? x : 0u;   // each key once
        }
      };
      ProbeGroup ring[PROBE_RING];
#pragma unroll
      for (int s2 = 0; s2 < PROBE_RING; ++s2) issue(ring[s2], s2);
      for (int it = 0; it < n; it += PROBE_RING) {
#pragma unroll
        for (int s2 = 0; s2 < PROBE_RING; ++s2) {
          if (it + s2 < n) fold(ring[s2], it + s2);
          issue(ring[s2], it + s2 + PROBE_RING);
        }
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
