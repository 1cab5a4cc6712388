// The step's main kernel (task page "Gated attention decode", section "What to
// compute"; window and causal rules from section "Shapes"): split, QK-norm and
// RoPE of the queries, the fp8 write of the new k/v rows, and split-K
// softmax(q . K^T / 8) . V over the paged FP8 cache for every block token and
// query head.  Work-groups take equal shares of all requests' key
// chunks (see attn_kernel) and write one partial (reference max, sum,
// unnormalised output) per (token, head) and segment; combine.hip merges them.
//
// Data path per 32-key chunk (one wave):
//  * cache rows come from an LDS copy of the split's table entries, so the
//    dependent index load never stalls the row loads;
//  * K rows: lane (n = lane%16, j = lane/16) loads 16 B of key n's row at
//    byte 16j (KV head 0) and 64+16j (KV head 1) -- the A operand of
//    S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (fp8 -> bf16 is exact);
//  * Q^T is block-diagonal: head n's column is zero on the other KV head's
//    dims, and q is carried as bf16 hi + lo (two MFMAs) so the product keeps
//    ~16 significant bits of q;
//  * the S^T tile leaves head n's scores for keys 4j..4j+3 (and 16+4j..) in
//    lane (n, j): exactly the B operand layout of O^T = V^T . P^T, so P needs
//    no data movement (P is carried as bf16 hi + lo as well);
//  * V^T is the A operand of that product: lane (n, j) loads 8 B (dims
//    8n..8n+7 of both KV heads) of the 8 keys it holds P for, and an 8x8 byte
//    transpose in registers turns them into 8 M-tiles (row n of M-tile mt =
//    byte 8n+mt of the V row);
//  * online softmax in base 2 (log2(e)/8 and kv_scale are folded into q).
//
// One 8-wave work-group per CU: two work-groups sharing a CU progress at
// unequal rates (the older one wins issue arbitration), so the younger one
// would finish alone.  Decode (L = 1): the 8 waves take interleaved chunks of
// a segment and merge their states in LDS.  Verify (L > 1): wave w owns block
// token w and walks every chunk of the segment (the re-reads of a row by the
// 8 waves hit the cache).
#include "device_common.h"
#include "launch.h"

namespace museattn {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int MAX_SPLIT_LDS = 4096;   // table entries cached per work-group
constexpr float RESCALE_SLACK = 8.0f;  // log2 units a stale reference max may lag

struct RowBuf {
  uint4 k[4];   // [tile*2 + kv head] 16 B of K row
  uint2 v[8];   // 8 B of V rows of the 8 keys this lane holds P for
};

struct TokState {
  f32x4 o[8];   // O^T accumulators, M-tile mt = bytes 8*row + mt of the V row
  float m;      // running max (log2 units), same in the 4 lanes of a head
  float l;      // this lane's share of the running sum
  int lo, hi;   // visible key positions of the token, inclusive
  bool live;
};

struct QOps {
  bf16x8 hi[4], lo[4];   // B operand of S^T per K-step
};

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t x, uint32_t y) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 4x4 byte transpose: y_k byte i = x_i byte k.
__device__ __forceinline__ void transpose4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                             uint32_t &y0, uint32_t &y1, uint32_t &y2,
                                             uint32_t &y3) {
  const uint32_t t0 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0b0 x1b0 x0b1 x1b1
  const uint32_t t1 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0b2 x1b2 x0b3 x1b3
  const uint32_t t2 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
  y0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  y1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  y2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  y3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Max / sum over the 4 lanes n, n+16, n+32, n+48 (one head's lanes).
__device__ __forceinline__ float head_max(float x) {
  int xi = __float_as_int(x);
  auto p = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
  xi = __float_as_int(x);
  auto q = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__int_as_float(q[0]), __int_as_float(q[1]));
}

__device__ __forceinline__ float head_sum(float x) {
  int xi = __float_as_int(x);
  auto p = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  x = __int_as_float(p[0]) + __int_as_float(p[1]);
  xi = __float_as_int(x);
  auto q = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __int_as_float(q[0]) + __int_as_float(q[1]);
}

__device__ __forceinline__ void load_rows(RowBuf &rb, const uint8_t *__restrict__ kc,
                                          const uint8_t *__restrict__ vc,
                                          const uint32_t *lrows, int n, int j) {
  const uint32_t k0 = lrows[n];
  const uint32_t k1 = lrows[16 + n];
  const uint4 va = *reinterpret_cast<const uint4 *>(lrows + 4 * j);
  const uint4 vb = *reinterpret_cast<const uint4 *>(lrows + 16 + 4 * j);
  const uint8_t *kp0 = kc + (uint64_t)k0 * ROW + 16 * j;
  const uint8_t *kp1 = kc + (uint64_t)k1 * ROW + 16 * j;
  rb.k[0] = *reinterpret_cast<const uint4 *>(kp0);
  rb.k[1] = *reinterpret_cast<const uint4 *>(kp0 + 64);
  rb.k[2] = *reinterpret_cast<const uint4 *>(kp1);
  rb.k[3] = *reinterpret_cast<const uint4 *>(kp1 + 64);
  const uint32_t vr[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    rb.v[i] = *reinterpret_cast<const uint2 *>(vc + (uint64_t)vr[i] * ROW + 8 * n);
}

template <int NT>
__device__ __forceinline__ void compute_chunk(const RowBuf &rb, int u0, int j,
                                              TokState (&ts)[NT], const QOps (&q)[NT]) {
  // K operands: tile t (keys 16t..16t+15), K-step kk = (KV head kk/2, 8-byte half kk%2)
  bf16x8 ka[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ka[t][0] = fp8x8_to_bf16(rb.k[2 * t].x, rb.k[2 * t].y);
    ka[t][1] = fp8x8_to_bf16(rb.k[2 * t].z, rb.k[2 * t].w);
    ka[t][2] = fp8x8_to_bf16(rb.k[2 * t + 1].x, rb.k[2 * t + 1].y);
    ka[t][3] = fp8x8_to_bf16(rb.k[2 * t + 1].z, rb.k[2 * t + 1].w);
  }
  // V operands: 8x8 byte transpose (key slot i x dim-byte mt) then fp8 -> bf16
  uint32_t tx[8], ty[8];
  transpose4x4(rb.v[0].x, rb.v[1].x, rb.v[2].x, rb.v[3].x, tx[0], tx[1], tx[2], tx[3]);
  transpose4x4(rb.v[0].y, rb.v[1].y, rb.v[2].y, rb.v[3].y, tx[4], tx[5], tx[6], tx[7]);
  transpose4x4(rb.v[4].x, rb.v[5].x, rb.v[6].x, rb.v[7].x, ty[0], ty[1], ty[2], ty[3]);
  transpose4x4(rb.v[4].y, rb.v[5].y, rb.v[6].y, rb.v[7].y, ty[4], ty[5], ty[6], ty[7]);
  bf16x8 vb[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) vb[mt] = fp8x8_to_bf16(tx[mt], ty[mt]);

#pragma unroll
  for (int tk = 0; tk < NT; ++tk) {
    TokState &st = ts[tk];
    if (!st.live) continue;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][kk], q[tk].hi[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][kk], q[tk].hi[kk], s1, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][kk], q[tk].lo[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][kk], q[tk].lo[kk], s1, 0, 0, 0);
    }
    float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    // only a chunk that straddles the token's visible range needs a mask
    if (u0 < st.lo || u0 + CHUNK - 1 > st.hi) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int u = u0 + (i >> 2) * 16 + 4 * j + (i & 3);
        if (u < st.lo || u > st.hi) sc[i] = -INFINITY;
      }
    }
    float cmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                       fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    cmax = head_max(cmax);
    // Lazy rescale: the reference max st.m only moves when some head's chunk
    // max exceeds it by more than RESCALE_SLACK (log2 units), so P <= 2^SLACK.
    // Any reference gives the same softmax; this one skips most rescales.
    if (__any(cmax > st.m + RESCALE_SLACK)) {
      const float mnew = fmaxf(st.m, cmax);
      const float alpha = mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(st.m - mnew);
      st.l *= alpha;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) st.o[mt] *= alpha;
      st.m = mnew;
    }
    const float muse = st.m == -INFINITY ? 0.0f : st.m;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(sc[i] - muse);
      st.l += pv[i];
    }
    bf16x8 ph, pl;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const f32x2 f = {pv[i], pv[i + 1]};
      const bf16x2 h = __builtin_convertvector(f, bf16x2);
      const bf16x2 r = __builtin_convertvector(f - __builtin_convertvector(h, f32x2), bf16x2);
      ph[i] = h[0]; ph[i + 1] = h[1];
      pl[i] = r[0]; pl[i + 1] = r[1];
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      st.o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[mt], ph, st.o[mt], 0, 0, 0);
      st.o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[mt], pl, st.o[mt], 0, 0, 0);
    }
  }
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
// theta = fp32(p) * inv_i with inv_i = base^(-i/32) rounded to fp32; sin/cos
// of that fp32 angle are taken in double so large positions keep full
// accuracy (task page "Gated attention decode", section "What to compute",
// the rope line; sliding layers only, section "Shapes").
__device__ __forceinline__ float2 rope_cs(float rope_base, int p, int i) {
  const float inv = (float)pow((double)rope_base, -(double)i / 32.0);
  const float th = (float)p * inv;
  double sd, cd;
  sincos((double)th, &sd, &cd);
  return make_float2((float)cd, (float)sd);
}

// Split and QK-norm of token t's query, RoPE on sliding layers, and the B
// operand of S^T = K . Q^T (task page "Gated attention decode", section "What
// to compute", first three lines of the listing).  Lane (n, j) owns dims
// 16j..16j+15 of head n: the head's rmsnorm is a sum over its 4 lanes, the
// RoPE partner (dim +-32) sits in lane (n, j ^ 2) = lane ^ 32.  K-step kk of
// the operand holds q[16j + 8(kk%2) + i] (i < 8) when head n belongs to KV
// head kk/2, else 0; q (times log2(e)/8 and kv_scale) is split into bf16
// hi + lo.  cs: the token's 32 (cos, sin) pairs in LDS (sliding only).
struct QIn {
  uint4 r0, r1;   // the lane's 16 bf16 values of q
};

__device__ __forceinline__ QIn load_q_in(const StepArgs &a, int t, int n, int j) {
  const uint16_t *src = a.qkv + (size_t)t * QKV_W + n * D + 16 * j;
  return QIn{*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 8)};
}

__device__ __forceinline__ void make_q(const StepArgs &a, const QIn &in, const f32x4 (&wv)[4],
                                       int j, int n, float qmul, const float2 *cs, QOps &qo) {
  const uint32_t raw[8] = {in.r0.x, in.r0.y, in.r0.z, in.r0.w, in.r1.x, in.r1.y, in.r1.z, in.r1.w};
  float x[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = __uint_as_float(raw[k] << 16);
    x[2 * k + 1] = __uint_as_float(raw[k] & 0xffff0000u);
  }
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) ss += x[k] * x[k];
  const float ms = head_sum(ss) * (1.0f / 64.0f);
  const float den = sqrtf(ms + a.eps);
  float y[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] = x[k] / den * wv[k >> 2][k & 3] * a.q_scale;
  if (a.sliding) {
    const bool low = j < 2;   // dims < 32: x_i c - x_{i+32} s ; else x_{i+32} c + x_i s
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int yi = __float_as_int(y[k]);
      const auto sw = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
      const float partner = __int_as_float(low ? sw[1] : sw[0]);
      const float2 c = cs[(16 * j + k) & 31];
      y[k] = low ? y[k] * c.x - partner * c.y : y[k] * c.x + partner * c.y;
    }
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float mul = (n >> 3) == (kk >> 1) ? qmul : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const f32x2 f = {y[8 * (kk & 1) + i] * mul, y[8 * (kk & 1) + i + 1] * mul};
      const bf16x2 h = __builtin_convertvector(f, bf16x2);
      const bf16x2 l = __builtin_convertvector(f - __builtin_convertvector(h, f32x2), bf16x2);
      qo.hi[kk][i] = h[0]; qo.hi[kk][i + 1] = h[1];
      qo.lo[kk][i] = l[0]; qo.lo[kk][i + 1] = l[1];
    }
  }
}

// The new k and v rows of the block tokens flagged in `own` (bit jt = token
// jt of request b, at position pos[jt]): k = rmsnorm(k) * w_k, rotated on
// sliding layers, then fp8(k / kv_scale) and fp8(v / kv_scale) into cache row
// row(b, p) (task page "Gated attention decode", section "What to compute",
// the cache line of the listing).  Wave 0/1: k head 0/1, wave 2/3: v head 0/1;
// lane = dim.  All tokens' inputs are loaded before any is used.
struct RowIn {
  float x[8];   // the lane's k or v value of each block token
  float wk;
};

__device__ __forceinline__ RowIn load_row_in(const StepArgs &a, int b) {
  const int wave = threadIdx.x >> 6, d = threadIdx.x & 63;
  const int off = (wave < 2 ? K_OFF : V_OFF) + (wave & 1) * D + d;
  RowIn in;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    const int t = b * a.L + (jt < a.L ? jt : a.L - 1);
    in.x[jt] = bf16_bits_to_f32(a.qkv[(size_t)t * QKV_W + off]);
  }
  in.wk = a.wk[d];
  return in;
}

__device__ __forceinline__ void write_new_rows(const StepArgs &a, int b, unsigned own,
                                               const int (&pos)[8], const float2 (*cs)[32],
                                               const RowIn &in) {
  const int wave = threadIdx.x >> 6, d = threadIdx.x & 63;
  const bool is_k = wave < 2;
  const int g = wave & 1;
  const float wk = in.wk;
  float x[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) x[jt] = in.x[jt];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    if (!((own >> jt) & 1u)) continue;   // uniform
    float y = x[jt];
    if (is_k) {
      const float ms = wave_sum(y * y) * (1.0f / 64.0f);
      y = y / sqrtf(ms + a.eps) * wk;
      if (a.sliding) {
        const int yi = __float_as_int(y);
        const auto sw = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
        const float partner = __int_as_float(d < 32 ? sw[1] : sw[0]);
        const float2 c = cs[jt][d & 31];
        y = d < 32 ? y * c.x - partner * c.y : y * c.x + partner * c.y;
      }
    }
    uint8_t *dst = (is_k ? a.k_cache : a.v_cache) + (uint64_t)cache_row(a, b, pos[jt]) * ROW +
                   g * D + d;
    *dst = to_e4m3(y / a.kv_scale);
  }
}

// Row buffers in flight per wave (decode).
#ifndef MUSEATTN_DECODE_NBUF
#define MUSEATTN_DECODE_NBUF 2
#endif

constexpr int PIECE_CHUNKS = MAX_SPLIT_LDS / CHUNK;   // chunks whose rows one LDS fill holds

// LDS row ids of a piece's keys kstart.. (clamped into [klo, khi]): the table
// loads are issued first (one memory round trip), the stores come later.
struct TableIn {
  int u[MAX_SPLIT_LDS / THREADS];
  int32_t unit[MAX_SPLIT_LDS / THREADS];
};

__device__ __forceinline__ void load_table_in(const StepArgs &a, int b, const KeyRange &r,
                                              int kstart, TableIn &in) {
  const int tid = threadIdx.x;
  const int shift = a.page_size == 1 ? 0 : 6;
  const int32_t *trow = a.table + (int64_t)b * a.table_stride;
#pragma unroll
  for (int it = 0; it < MAX_SPLIT_LDS / THREADS; ++it) {
    const int v = kstart + tid + it * THREADS;
    in.u[it] = v < r.klo ? r.klo : (v > r.khi ? r.khi : v);
  }
#pragma unroll
  for (int it = 0; it < MAX_SPLIT_LDS / THREADS; ++it) in.unit[it] = trow[in.u[it] >> shift];
}

__device__ __forceinline__ void store_table(const StepArgs &a, const TableIn &in, uint32_t *lrows) {
  const int tid = threadIdx.x;
  const int shift = a.page_size == 1 ? 0 : 6;
  const uint32_t units = (uint32_t)(a.num_rows >> shift);
#pragma unroll
  for (int it = 0; it < MAX_SPLIT_LDS / THREADS; ++it) {
    uint32_t un = (uint32_t)in.unit[it];
    un = un < units ? un : units - 1;
    lrows[tid + it * THREADS] = (un << shift) + (uint32_t)(in.u[it] & (a.page_size - 1));
  }
}

struct Lds {
  uint32_t lrows[MAX_SPLIT_LDS];
  float2 cs[8][32];          // RoPE (cos, sin) per block token and pair
  float sm_o[WAVES][HQ][D];
  float sm_m[WAVES][HQ];
  float sm_l[WAVES][HQ];
  int pref[MAX_BATCH + 1];
  int scan[THREADS];
  int req_len[MAX_BATCH];    // seq_lens[b], kept from the plan
  int req_p0[MAX_BATCH];     // positions[b * L] (sliding layers)
};

// One segment: chunks [x, y) of request b's key range (chunk i = keys
// kbase + 32i ..), processed by the whole work-group, leaving one partial per
// (token, head) in slot `slot`.
template <int MODE, int NT, int NBUF>
__device__ __forceinline__ void process_segment(const StepArgs &a, int b, const KeyRange &r, int x,
                                                int y, int slot, Lds &sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const float qmul = a.kv_scale * (LOG2E / 8.0f);
  const int nseg = y - x;
  const int npieces = (nseg + PIECE_CHUNKS - 1) / PIECE_CHUNKS;
  auto piece_x = [&](int pc) { return x + (int)((int64_t)pc * nseg / npieces); };

  // One batch of loads for everything the segment starts with: positions, the
  // first piece's table entries, the tokens' q rows and norm weights, and the
  // inputs of the new k/v rows.
  int pos[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) pos[jt] = a.positions[b * a.L + (jt < a.L ? jt : a.L - 1)];
  TableIn tin;
  load_table_in(a, b, r, r.kbase + x * CHUNK, tin);
  QIn qin[NT];
#pragma unroll
  for (int tk = 0; tk < NT; ++tk) {
    const int jt = MODE == 0 ? 0 : wave + WAVES * tk;
    qin[tk] = load_q_in(a, b * a.L + (jt < a.L ? jt : 0), n, j);
  }
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(a.wq + 16 * j);
  const f32x4 wv[4] = {w4[0], w4[1], w4[2], w4[3]};
  const RowIn rin = load_row_in(a, b);
  __builtin_amdgcn_sched_barrier(0);

  __syncthreads();   // the previous segment is done with sh.cs and sh.lrows
  if (a.sliding) {
    if (tid < a.L * 32) sh.cs[tid >> 5][tid & 31] = rope_cs(a.rope_base, a.positions[b * a.L + (tid >> 5)], tid & 31);
    __syncthreads();
  }
  store_table(a, tin, sh.lrows);
  TokState ts[NT];
  QOps qo[NT];
#pragma unroll
  for (int tk = 0; tk < NT; ++tk) {
    const int jt = MODE == 0 ? 0 : wave + WAVES * tk;
    ts[tk].live = jt < a.L;
    const int jq = ts[tk].live ? jt : 0;
    int p = pos[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) p = jq == k ? pos[k] : p;
    ts[tk].hi = p < r.khi ? p : r.khi;
    ts[tk].lo = a.sliding ? p - (WINDOW - 1) : 0;
    ts[tk].m = -INFINITY;
    ts[tk].l = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) ts[tk].o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    make_q(a, qin[tk], wv, j, n, qmul, sh.cs[jq], qo[tk]);
  }
  bool any_live = false;
#pragma unroll
  for (int tk = 0; tk < NT; ++tk) any_live |= ts[tk].live;
  // New rows of the block tokens whose key falls in this segment: only this
  // work-group reads them, so a workgroup release before the barrier orders
  // the writes before its own loads.
  unsigned owned = 0;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    const int p = pos[jt];
    const bool in = jt < a.L && p >= r.klo && p <= r.khi &&
                    (p - r.kbase) / CHUNK >= x && (p - r.kbase) / CHUNK < y;
    owned |= in ? 1u << jt : 0u;
  }
  if (owned && wave < 4) write_new_rows(a, b, owned, pos, sh.cs, rin);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();

  for (int pc = 0; pc < npieces; ++pc) {
    const int px = piece_x(pc), py = piece_x(pc + 1);
    const int nchunks = py - px;
    const int kstart = r.kbase + px * CHUNK;
    if (pc > 0) {
      __syncthreads();   // every wave is done with the previous rows
      TableIn tn;
      load_table_in(a, b, r, kstart, tn);
      __builtin_amdgcn_sched_barrier(0);
      store_table(a, tn, sh.lrows);
      __syncthreads();
    }

    // This wave's chunks of the piece: c0, c0 + cstep, ... (nloc of them).  In
    // the steady state every load is unconditional -- chunk indices past the
    // end are clamped to the last chunk -- so the compiler can count the loads
    // in flight and wait only for the buffer it is about to use.
    const int c0 = MODE == 0 ? wave : 0;
    const int cstep = MODE == 0 ? WAVES : 1;
    const int nloc = nchunks > c0 ? (nchunks - c0 + cstep - 1) / cstep : 0;
    if (any_live && nloc > 0) {
      const int last = nloc - 1;
      RowBuf buf[NBUF];
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        const int i = k < last ? k : last;
        load_rows(buf[k], a.k_cache, a.v_cache, sh.lrows + (c0 + i * cstep) * CHUNK, n, j);
      }
      int i = 0;
      for (; i + NBUF <= nloc; i += NBUF) {
#pragma unroll
        for (int k = 0; k < NBUF; ++k) {
          compute_chunk<NT>(buf[k], kstart + (c0 + (i + k) * cstep) * CHUNK, j, ts, qo);
          int inext = i + k + NBUF;
          inext = inext < last ? inext : last;
          load_rows(buf[k], a.k_cache, a.v_cache, sh.lrows + (c0 + inext * cstep) * CHUNK, n, j);
        }
      }
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k)
        if (i + k < nloc)
          compute_chunk<NT>(buf[k], kstart + (c0 + (i + k) * cstep) * CHUNK, j, ts, qo);
    }
  }

  // Lane (n, j) holds O^T of head n at V-row bytes 8(4j + r) + mt, r < 4: KV head
  // j/2, dims 32(j%2) + 8r + mt.  Only lanes whose KV head is head n's own hold
  // meaningful values.
  const bool own = (j >> 1) == (n >> 3);
  const int dbase = 32 * (j & 1);
  if (MODE == 0) {
    const float lsum = head_sum(ts[0].l);
    if (j == 0) {
      sh.sm_m[wave][n] = ts[0].m;
      sh.sm_l[wave][n] = lsum;
    }
    if (own) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float *dst = &sh.sm_o[wave][n][dbase + 8 * rr];
        *reinterpret_cast<f32x4 *>(dst) =
            f32x4{ts[0].o[0][rr], ts[0].o[1][rr], ts[0].o[2][rr], ts[0].o[3][rr]};
        *reinterpret_cast<f32x4 *>(dst + 4) =
            f32x4{ts[0].o[4][rr], ts[0].o[5][rr], ts[0].o[6][rr], ts[0].o[7][rr]};
      }
    }
    __syncthreads();
    // merge the waves: thread -> (head h, dims d2, d2 + 1)
    const int h = tid >> 5, d2 = (tid & 31) * 2;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.sm_m[w][h]);
    f32x2 o = {0.f, 0.f};
    float lt = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float sc = __builtin_amdgcn_exp2f(sh.sm_m[w][h] - M);
        lt += sc * sh.sm_l[w][h];
        o += sc * *reinterpret_cast<const f32x2 *>(&sh.sm_o[w][h][d2]);
      }
    }
    const size_t e = (size_t)slot * HQ + h;   // L = 1
    *reinterpret_cast<f32x2 *>(a.part_o + e * D + d2) = o;
    if ((tid & 31) == 0) {
      a.part_ml[e * 2] = M;
      a.part_ml[e * 2 + 1] = lt;
    }
  } else {
#pragma unroll
    for (int tk = 0; tk < NT; ++tk) {
      const float lsum = head_sum(ts[tk].l);
      if (!ts[tk].live) continue;
      const int jt = wave + WAVES * tk;
      const size_t e = ((size_t)slot * a.L + jt) * HQ + n;
      if (j == 0) {
        a.part_ml[e * 2] = ts[tk].m;
        a.part_ml[e * 2 + 1] = lsum;
      }
      if (own) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float *dst = a.part_o + e * D + dbase + 8 * rr;
          *reinterpret_cast<f32x4 *>(dst) =
              f32x4{ts[tk].o[0][rr], ts[tk].o[1][rr], ts[tk].o[2][rr], ts[tk].o[3][rr]};
          *reinterpret_cast<f32x4 *>(dst + 4) =
              f32x4{ts[tk].o[4][rr], ts[tk].o[5][rr], ts[tk].o[6][rr], ts[tk].o[7][rr]};
        }
      }
    }
  }
}

// The attention kernel.  Every work-group derives the same plan from the
// device-side sequence lengths: request b spans chunks [pref[b], pref[b+1]) of
// the concatenated chunk space, and work-group w takes an equal contiguous
// share of it (counting each request start as seg_cost chunks), so no
// work-group idles while another still has a long split.
// A share that crosses request boundaries is processed one segment per
// request; segment (w, b) writes its partial to slot w + b (slots are unique
// because both w and b grow along the chunk space).  The combine kernel then
// merges each request's slots.
template <int MODE, int NT, int NBUF>
__global__ __launch_bounds__(THREADS, 2) void attn_kernel(StepArgs a) {
  __shared__ __attribute__((aligned(16))) Lds sh;
  const int tid = threadIdx.x;

  // chunk-count prefix sums over the requests (RPT per thread, B <= 1024)
  constexpr int RPT = MAX_BATCH / THREADS;
  int cnt[RPT], sum = 0;
  {
    // lengths (and, on sliding layers, first positions) of the thread's
    // requests, loaded as one batch
    int sl[RPT], p0[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int b = RPT * tid + k < a.B ? RPT * tid + k : a.B - 1;
      sl[k] = a.seq_lens[b];
      p0[k] = a.sliding ? a.positions[b * a.L] : 0;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      cnt[k] = RPT * tid + k < a.B ? request_chunks(range_from(a, sl[k], p0[k])) : 0;
      sum += cnt[k];
      sh.req_len[RPT * tid + k] = sl[k];
      sh.req_p0[RPT * tid + k] = p0[k];
    }
  }
  sh.scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < THREADS; off <<= 1) {
    const int v = tid >= off ? sh.scan[tid - off] : 0;
    __syncthreads();
    sh.scan[tid] += v;
    __syncthreads();
  }
  {
    int run = sh.scan[tid] - sum;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int b = RPT * tid + k;
      if (b < a.B) sh.pref[b] = run;
      run += cnt[k];
    }
    if (tid == THREADS - 1) sh.pref[a.B] = sh.scan[THREADS - 1];
  }
  __syncthreads();
  // Cost space: request b occupies seg_cost units (its segment start-up, in
  // chunk-equivalents) followed by its chunks, so request b starts at cost
  // Q_b = pref[b] + b * seg_cost.  Work-groups take equal cost shares; one
  // whose share covers a request start gets correspondingly fewer chunks.
  const int pen = a.seg_cost;
  const int64_t Ct = (int64_t)sh.pref[a.B] + (int64_t)a.B * pen;
  const int w = blockIdx.x;
  const int G = Ct < a.work_groups ? (int)Ct : a.work_groups;
  if (w == 0) {
    // the plan, for the combine kernel: chunk prefix sums and work-groups used
    for (int i = tid; i <= a.B; i += THREADS) a.plan[i] = sh.pref[i];
    if (tid == 0) a.plan[a.B + 1] = G;
  }
  if (w >= G) return;   // uniform over the work-group
  const int64_t cb = (int64_t)w * Ct / G, ce = (int64_t)(w + 1) * Ct / G;
  auto cost_of = [&](int bb) { return (int64_t)sh.pref[bb] + (int64_t)bb * pen; };
  int b = 0;
  {
    int hi = a.B - 1;
    while (b < hi) {   // largest b whose cost range starts at or before cb
      const int mid = (b + hi + 1) >> 1;
      if (cost_of(mid) <= cb) b = mid; else hi = mid - 1;
    }
  }
  for (; b < a.B && cost_of(b) < ce; ++b) {
    const int64_t q0 = cost_of(b) + pen;            // cost of chunk 0 of request b
    const int64_t nb = sh.pref[b + 1] - sh.pref[b];
    const int64_t xs = cb - q0, ys = ce - q0;
    const int x = (int)(xs > 0 ? xs : 0);
    const int y = (int)(ys < nb ? ys : nb);
    if (y <= x) continue;
    const KeyRange r = range_from(a, sh.req_len[b], sh.req_p0[b]);
    process_segment<MODE, NT, NBUF>(a, b, r, x, y, w + b, sh);
  }
}

void launch_attn(const StepArgs &a, hipStream_t stream) {
  const dim3 grid(a.work_groups), block(THREADS);
  if (a.L == 1)
    hipLaunchKernelGGL((attn_kernel<0, 1, MUSEATTN_DECODE_NBUF>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_kernel<1, 1, 2>), grid, block, 0, stream, a);
}

}  // namespace museattn

