// Shared definitions of the gfx950 kernels of libmuseattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace museattn {

constexpr int HQ = 16;       // query heads per shard
constexpr int HKV = 2;       // KV heads per shard
constexpr int D = 64;        // head dim
constexpr int GROUP = 8;     // query heads per KV head; head h reads KV head h / 8
constexpr int QKV_W = 2304;  // fused row: [q 16x64 | k 2x64 | v 2x64 | gate 16x64]
constexpr int K_OFF = 1024, V_OFF = 1152, G_OFF = 1280;
constexpr int ROW = 128;     // bytes of one cache row (2 KV heads x 64 E4M3 bytes)
constexpr int WINDOW = 2048; // sliding window, the query's own position included
constexpr int CHUNK = 32;    // keys per step of the attention kernel's inner loop
constexpr int WAVES = 8;     // waves per attention work-group (one work-group per CU)
constexpr int THREADS = 64 * WAVES;
constexpr int MAX_BATCH = 1024;   // requests per call (prefix sums live in LDS)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Everything one step's kernels read, passed by value.
struct StepArgs {
  const uint16_t *qkv;     // bf16 bits [T][2304]
  const int32_t *positions;
  const int32_t *table;
  const int32_t *seq_lens;
  uint8_t *k_cache;
  uint8_t *v_cache;
  uint16_t *out;           // bf16 bits [T][1024]
  const float *wq, *wk, *wo;
  int *plan;               // [B + 2]: chunk prefix sums of the requests, then the
                           // work-groups used (written by attention work-group 0)
  float *part_ml;          // [slot][L][16][2] (reference max in log2 units, sum)
  float *part_o;           // [slot][L][16][64] unnormalised partial outputs
  int64_t num_rows;
  float kv_scale, eps, q_scale;
  float rope_inv[32];      // RoPE inverse frequencies fp32(rope_base^(-i/32)), pair i
  int B, L, table_stride, max_seq_len, page_size, sliding;
  int work_groups;         // attention work-groups launched (each takes an equal
                           // share of all requests' key chunks)
  int seg_cost;            // chunk-equivalents one segment start-up costs
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Cache row of request b's key position u (u already clamped into the valid
// key range).  Page (or row) ids are clamped into the pool so that no table
// value can address memory outside it.
__device__ __forceinline__ uint32_t cache_row(const StepArgs &a, int b, int u) {
  const int ps = a.page_size;
  const uint32_t units = (uint32_t)(a.num_rows / ps);
  uint32_t unit = (uint32_t)a.table[(int64_t)b * a.table_stride + u / ps];
  unit = unit < units ? unit : units - 1;
  return unit * (uint32_t)ps + (uint32_t)(u % ps);
}

// The union key range of request b's block tokens.  khi = seq_len - 1; klo =
// 0 on full layers, first token's position - 2047 on sliding ones.  kbase is
// klo rounded down to a whole CHUNK.
struct KeyRange {
  int klo, khi, kbase;
};

// The key range from a request's length and its first block token's position.
__device__ __forceinline__ KeyRange range_from(const StepArgs &a, int sl, int p0) {
  sl = sl < 0 ? 0 : (sl > a.max_seq_len ? a.max_seq_len : sl);
  KeyRange r;
  r.khi = sl - 1;
  r.klo = 0;
  if (a.sliding) {
    p0 = p0 < 0 ? 0 : (p0 > a.max_seq_len - 1 ? a.max_seq_len - 1 : p0);
    r.klo = p0 - (WINDOW - 1);
    r.klo = r.klo < 0 ? 0 : r.klo;
  }
  r.kbase = r.klo & ~(CHUNK - 1);
  return r;
}

// Chunks (of CHUNK keys, from kbase) that request b's key range spans.
__device__ __forceinline__ int request_chunks(const KeyRange &r) {
  return r.khi < r.klo ? 0 : (r.khi + 1 - r.kbase + CHUNK - 1) / CHUNK;
}

// Sum over the 64 lanes of a wave, result in every lane: DPP steps inside each
// 16-lane row (xor 1, xor 2, half-row mirror, row mirror), then the gfx950
// row swaps across rows.  VALU only, no LDS round trip.
#define MUSEATTN_DPP(x, ctrl) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), 0xf, 0xf, false))

__device__ __forceinline__ float wave_sum(float x) {
  x += MUSEATTN_DPP(x, 0xB1);    // quad_perm [1,0,3,2]
  x += MUSEATTN_DPP(x, 0x4E);    // quad_perm [2,3,0,1]
  x += MUSEATTN_DPP(x, 0x141);   // row_half_mirror
  x += MUSEATTN_DPP(x, 0x140);   // row_mirror
  int xi = __float_as_int(x);
  auto p = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = __int_as_float(p[0]) + __int_as_float(p[1]);
  xi = __float_as_int(x);
  auto q = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __int_as_float(q[0]) + __int_as_float(q[1]);
}

// Cost unit c of C spread over G work-groups (work-group w owns units
// [floor(w C / G), floor((w + 1) C / G))) belongs to work-group
// floor(((c + 1) G - 1) / C).
__device__ __forceinline__ int wg_of_chunk(int64_t c, int64_t C, int G) {
  return (int)(((c + 1) * G - 1) / C);
}

// Sum over each 16-lane row (DPP only).
__device__ __forceinline__ float row16_sum(float x) {
  x += MUSEATTN_DPP(x, 0xB1);
  x += MUSEATTN_DPP(x, 0x4E);
  x += MUSEATTN_DPP(x, 0x141);
  x += MUSEATTN_DPP(x, 0x140);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, MUSEATTN_DPP(x, 0xB1));
  x = fmaxf(x, MUSEATTN_DPP(x, 0x4E));
  x = fmaxf(x, MUSEATTN_DPP(x, 0x141));
  x = fmaxf(x, MUSEATTN_DPP(x, 0x140));
  int xi = __float_as_int(x);
  auto p = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
  xi = __float_as_int(x);
  auto q = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__int_as_float(q[0]), __int_as_float(q[1]));
}

}  // namespace museattn
