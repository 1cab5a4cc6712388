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
constexpr int PREFILL_TB = 16;    // block tokens per plan unit when L > 8 (prefill)
constexpr int MAX_L = 16384;      // block tokens per request
constexpr int MAX_UNITS = 4096;   // plan units (B * ceil(L / 16)) of a prefill call

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Loads marked non-temporal (the "nt" cache policy): the line is read for
// this access alone and is not kept for reuse.  For rows that one step reads
// once, from a working set far larger than the caches, this gathers faster
// than an ordinary load (which also fills the caches).
__device__ __forceinline__ uint4 load_nt16(const uint8_t *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt8(const uint8_t *p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  return make_uint2(v.x, v.y);
}

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
  int end_cost;            // and the unit's end (verify: its new rows)
  // Plan units: request b's block tokens in groups of tb (unit u = b * nblk +
  // blk holds tokens blk*tb ..); one group per request (tb = L) up to L = 8.
  int tb, nblk, nunits;
  uint64_t *ts;            // phase timestamps (MUSEATTN_PHASE_TIMES builds), else null
};

// Per-phase timestamps, compiled in only with MUSEATTN_PHASE_TIMES (an
// instrumented build of the library): thread 0 of a work-group stores the
// GPU's 100 MHz real-time counter, or a count, into one slot of its row of
// a.ts with an ordinary vector store.  Attention work-group w owns slots
// [w * TS_SLOTS, (w + 1) * TS_SLOTS); combine work-group c owns the two
// slots at work_groups * TS_SLOTS + 2c (entry, exit).
constexpr int TS_SLOTS = 12;
enum TsSlot {
  TS_ENTRY = 0,      // first instruction
  TS_PLAN = 1,       // the plan (prefix sums over the units) is in LDS
  TS_SETUP = 2,      // first segment: loads returned, row ids and q in place
  TS_STREAM = 3,     // first segment: every key chunk processed
  TS_PARTIAL = 4,    // first segment: partials written
  TS_EXIT = 5,       // last instruction
  TS_SEGMENTS = 6,   // segments processed (a count)
  TS_ISSUED = 7,     // first segment: its batch of loads issued
  TS_TABLE = 8,      // first segment: its row ids stored in LDS (the loads are back)
  TS_QREADY = 9,     // first segment: q operands (and any new rows) done, before the barrier
  TS_SEG2_START = 10,   // second segment (if any): entered
  TS_SEG2_SETUP = 11    // second segment: set-up done (its code is warm by now)
};
#ifdef MUSEATTN_PHASE_TIMES
__device__ __forceinline__ void stamp(const StepArgs &a, int slot, bool on = true) {
  if (on && threadIdx.x == 0)
    a.ts[(size_t)blockIdx.x * TS_SLOTS + slot] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void stamp_count(const StepArgs &a, int slot, uint64_t v) {
  if (threadIdx.x == 0) a.ts[(size_t)blockIdx.x * TS_SLOTS + slot] = v;
}
__device__ __forceinline__ void stamp_combine(const StepArgs &a, int which) {
  if (threadIdx.x == 0)
    a.ts[(size_t)a.work_groups * TS_SLOTS + 2 * (size_t)blockIdx.x + which] =
        __builtin_amdgcn_s_memrealtime();
}
#else
__device__ __forceinline__ void stamp(const StepArgs &, int, bool = true) {}
__device__ __forceinline__ void stamp_count(const StepArgs &, int, uint64_t) {}
__device__ __forceinline__ void stamp_combine(const StepArgs &, int) {}
#endif

// Request and token group of plan unit u.
__device__ __forceinline__ void unit_of(const StepArgs &a, int u, int &b, int &blk) {
  b = u / a.nblk;
  blk = u - b * a.nblk;
}

// Key positions of unit u's union range end at this length (its last token's
// position + 1): seq_len_b - L + min(L, (blk + 1) tb).
__device__ __forceinline__ int unit_len(const StepArgs &a, int seq_len, int blk) {
  const int end = (blk + 1) * a.tb;
  return seq_len - a.L + (end < a.L ? end : a.L);
}

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
  const int shift = a.page_size == 1 ? 0 : 6;   // page size 1 or 64
  const uint32_t units = (uint32_t)(a.num_rows >> shift);
  uint32_t unit = (uint32_t)a.table[(int64_t)b * a.table_stride + (u >> shift)];
  unit = unit < units ? unit : units - 1;
  return (unit << shift) + (uint32_t)(u & (a.page_size - 1));
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

// floor(n / d) for 0 <= n < 2^50 and 0 < d < 2^31.  gfx950 has no 64-bit
// integer divide: the compiler's sequence is ~130 scalar instructions, which
// every wave of a work-group runs on the CU's one scalar unit.  Here n times
// the double reciprocal of d (v_rcp_f64, a few ulp: within two of the true
// quotient for such operands) is corrected to the exact floor with integer
// products.
__device__ __forceinline__ int64_t div_floor(int64_t n, int64_t d) {
  int64_t q = (int64_t)((double)n * __builtin_amdgcn_rcp((double)d));
  // at most two steps either way; straight-line selects, no loop (a loop's
  // block boundaries would keep the scheduler from moving loads across it)
  q -= q * d > n ? 1 : 0;
  q -= q * d > n ? 1 : 0;
  q += (q + 1) * d <= n ? 1 : 0;
  q += (q + 1) * d <= n ? 1 : 0;
  return q;
}

// Cost unit c of C spread over G work-groups (work-group w owns units
// [floor(w C / G), floor((w + 1) C / G))) belongs to work-group
// floor(((c + 1) G - 1) / C).
__device__ __forceinline__ int wg_of_chunk(int64_t c, int64_t C, int G) {
  return (int)div_floor((c + 1) * G - 1, C);
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

// E4M3FN byte of x (OCP format: bias 7, max 448, no infinities), round to
// nearest even, saturating.  The gfx950 converter rounds to nearest even but
// turns magnitudes past the last rounding interval into NaN, so values are
// clamped to +-448 first; NaN stays NaN.
__device__ __forceinline__ uint8_t to_e4m3(float x) {
  if (fabsf(x) > 448.0f) x = copysignf(448.0f, x);
  const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false);
  return (uint8_t)(packed & 0xff);
}

// RoPE factors of one block token: pair i (dims i, i+32) turns by
// theta = fp32(p) * inv_i with inv_i = base^(-i/32) rounded to fp32 (a table
// the host fills once per call); sin/cos of that fp32 angle are taken in
// double so large positions keep full accuracy (task page "Gated attention
// decode", section "What to compute", the rope line; sliding layers only,
// section "Shapes").
//
// The table is read from the kernel's argument block, whose first member is
// the StepArgs (a per-lane index into the by-value argument itself would make
// the compiler copy it to scratch).
__device__ __forceinline__ float rope_inv(int i) {
  const char *args = (const char *)__builtin_amdgcn_kernarg_segment_ptr();
  return reinterpret_cast<const float *>(args + offsetof(StepArgs, rope_inv))[i];
}

// (cos, sin) of position p for a pair whose inverse frequency is inv.
__device__ __forceinline__ float2 rope_cs_inv(int p, float inv) {
  const float th = (float)p * inv;
  double sd, cd;
  sincos((double)th, &sd, &cd);
  return make_float2((float)cd, (float)sd);
}

__device__ __forceinline__ float2 rope_cs(int p, int i) { return rope_cs_inv(p, rope_inv(i)); }

}  // namespace museattn
