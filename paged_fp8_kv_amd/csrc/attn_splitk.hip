// The step's main kernel (task page "Gated attention decode", section "What to
// compute"; window and causal rules from section "Shapes"): split, QK-norm and
// RoPE of the queries, the fp8 write of the new k/v rows, and split-K
// softmax(q . K^T / 8) . V over the paged FP8 cache for every block token and
// query head.  Work-groups take equal shares of all requests' key
// chunks (see attn_kernel) and write one partial (reference max, sum,
// unnormalised output) per (token, head) and segment; combine.hip merges them.
//
// Decode data path per 32-key chunk (one wave):
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
// a segment and merge their states in LDS.  Verify and prefill blocks (L >=
// 2): the block tokens x 8 heads of a KV group form a dense contraction on
// fp16 MFMA over K/V staged in LDS (see the block section below); waves split
// the KV heads, the column tiles and (verify) the sub-chunks.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace museattn {

constexpr float LOG2E = 1.4426950408889634f;

// A partial's store.  NT: non-temporal, for decode steps that may read more
// than 512 MB of rows and verify blocks from 4 MB: their partials are read
// once, by the merge kernel, and need not sit in L2 at the kernel's end
// (decode B 32: step 116.7-117.7 -> 115.8-116.2 us).  Smaller steps keep
// ordinary stores, whose merge finds them in L2 (paged decode B 16: 58.3-58.4
// vs 58.9-59.2 us; sliding decode B 1: 11.6-11.7 vs 12.0-12.1 us).
template <bool NT = false, class T>
__device__ __forceinline__ void part_store(T *p, T v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}
constexpr int MAX_SPLIT_LDS = 4096;   // table entries cached per work-group
// log2 units a stale reference max may lag: P <= 2^15 stays inside fp16's
// range (65504) in the block products
constexpr float RESCALE_SLACK = 15.0f;

struct RowBuf {
  uint4 k[4];   // [tile*2 + kv head] 16 B of K row
  uint2 v[8];   // 8 B of V rows of the 8 keys this lane holds P for
};

struct TokState {
  f32x4 o[8];   // O^T accumulators, M-tile mt = bytes 8*row + mt of the V row
  float m;      // running max (log2 units), same in the 4 lanes of a head
  float l;      // this lane's share of the running sum
  int lo, hi;   // visible key positions of the token, inclusive
};

// Decode: the B operand of S^T per K-step kk (hi and lo parts), one copy in
// LDS for the work-group's 8 waves (they all serve the same token): [kk][hi,
// lo][lane].
struct QOps {
  bf16x8 op[4][2][64];
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

// Blocks: the same 8 codes in fp16 (also exact: every E4M3 value is an fp16
// value).
__device__ __forceinline__ f16x8 fp8x8_to_f16(uint32_t x, uint32_t y) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y, 1.0f, true);
  f16x8 r;
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

// NTV: V rows by non-temporal loads.  Each V load instruction reads 4 whole
// rows (16 lanes x 8 bytes each); a K load reads half of each of 16 rows, the
// other half coming from the next instruction, which finds the line in L2
// only if the first one kept it -- so K keeps ordinary loads.
template <bool NTV>
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
  for (int i = 0; i < 8; ++i) {
    const uint8_t *vp = vc + (uint64_t)vr[i] * ROW + 8 * n;
    rb.v[i] = NTV ? load_nt8(vp) : *reinterpret_cast<const uint2 *>(vp);
  }
}

__device__ __forceinline__ void compute_chunk(const RowBuf &rb, int u0, int lane, TokState &st,
                                              const QOps &q) {
  const int j = lane >> 4;
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

  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bf16x8 qh = q.op[kk][0][lane], ql = q.op[kk][1][lane];
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][kk], qh, s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][kk], qh, s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][kk], ql, s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][kk], ql, s1, 0, 0, 0);
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

// Verify and prefill blocks (L >= 2): per KV head g, a dense contraction of
// the block's (token, head) columns with the keys.  Column tile ct holds
// tokens 2ct and 2ct + 1 of the unit (lane column n: token 2ct + n/8, head
// 8g + n%8).  The work-group moves through a segment in steps of 64 keys (two
// 32-key sub-chunks) that its 8 waves share:
//  * staging: lanes 0-31 of each wave load 32 B of a K row, lanes 32-63 32 B
//    of a V row (stage_map), so 4 lanes read one whole 128-B row; the bytes
//    are converted to fp16 (exactly) once for the work-group and written,
//    key-major, into one of two LDS stage buffers (K chunks swizzled, V rows
//    padded, so that no LDS pass meets a bank twice).  The
//    loads run BLOCK_PREFETCH steps ahead in registers; one barrier per step.
//  * S^T (32 keys x 16 columns) per sub-chunk and column tile: 2 key tiles x
//    2 K-steps of v_mfma_f32_16x16x32_f16; A = K rows from LDS (K-step kk:
//    dims 32kk + 8j..+7 in lane (n, j)), B = Q^T from registers in fp16 (11
//    significant bits of q, scaled by a power of two if it would overflow).
//  * S^T leaves column n's scores for keys 4j..4j+3 (key tile 0) and
//    16+4j..16+4j+3 (key tile 1) in lane (n, j): the B operand layout of
//    O^T = V^T . P^T, so P stays in place, rounded to fp16.
//  * V^T tiles come from the row-major stage through the gfx950 transposing
//    LDS read (ds_read_b64_tr_b16): within a 16-lane group, lane s names 4
//    dims of key k0 + s/4 and lane i receives dim i of those 4 keys.
//  * online softmax in base 2 with decode's lazy reference max.
// Verify (L <= 8, up to 4 column tiles): wave w takes KV head w % 2, column
// tiles 2h and 2h + 1 with h = (w / 2) % 2, and sub-chunk w / 4 of each step;
// the two sub-chunk halves merge in LDS.  Prefill (token groups of 16, 8
// column tiles per KV head): wave w takes KV head w % 2, column tiles 2(w/2)
// and 2(w/2) + 1, and both sub-chunks of each step.
constexpr int STAGE_KEYS = 64;
// LDS passes on gfx950 (measured with the bank-conflict counter, one pair of
// active lanes at a time): ds_read_b128 serves 16 lanes per pass, lanes
// {0-3, 12-15, 20-23, 24-27}, {4-7, 8-11, 16-19, 28-31} and the same sets + 32,
// over 64 banks of 4 B; ds_write_b128 serves 8 consecutive lanes per pass over
// 32 banks.  A read pass is conflict-free when its 16 lanes hit 16 distinct
// 16-B bank quads (address / 16 mod 16), a write pass when its 8 lanes hit
// distinct quads mod 8.
// K stage: 256-B rows (2 heads x 64 fp16), 16-B chunk c of key r at slot
// c ^ (r % 16).  The operand reads (keys n = 0..15 of a tile, chunk cb + j
// with cb a multiple of 4) then hit quads cb ^ j ^ n, distinct in every read
// pass; the stores (keys r..r+7, one chunk) hit quads c ^ (r % 8) mod 8.  A
// plain padded stride meets only one of the two (272 B: the reads conflict;
// 288 B: the stores do).
constexpr int KROW = 256;   // LDS bytes per key of the K stage
constexpr int VROW = 288;   // of the V stage: + 32 B (see stage_map for its chunk order)

struct Stage {
  uint8_t k[STAGE_KEYS * KROW];
  uint8_t v[STAGE_KEYS * VROW];
};

struct BlockState {
  // O^T [dim tile dt][column tile c]: element r of lane (n, j) = dim 16dt + 4j + r.
  // Tile 4 is ones . P^T: every element holds the column's running sum of P.
  f32x4 o[5][2];
  f32x4 negm[2];   // -m (0 while m = -inf), the accumulator the scores start from
  float m[2];      // the column's reference max (log2 units)
  int lo[2], hi[2];   // visible key range of the lane column's token, inclusive
  int ulo[2], uhi[2]; // wave-uniform: keys [ulo, uhi] are visible to every live column
  float thr[2];       // the reference moves once the tile max passes this:
                      // -inf while the column has no reference, else the slack
  int e[2];           // q of the lane column is held as q * 2^-e in fp16 (e = 0
                      // unless |q| * qmul reaches 2^15)
  bool scaled;        // some column of the wave has e > 0 (wave-uniform)
  f16x8 ones;         // the all-ones operand of the P-sum tile
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One step's staged bytes between their load and their LDS store.
struct StageIn {
  uint4 x[2];
};

// Which 32 bytes thread t stages: wave w takes keys 8w..8w+7 of the step.
// Lanes 0-31 take K rows (key 8w + l%8, part [0, 2, 1, 3][l/8]); lanes 32-63
// take V rows, each group of 8 lanes 4 keys x 2 adjacent parts.  A part is 32
// fp8 bytes = 64 fp16 bytes = 4 chunks of 16 B, written one chunk per
// ds_write_b128.  In the V stage an odd part's chunk q sits at slot (q - 1) %
// 4; with this order the 8 (or 16) lanes an LDS pass serves hit distinct
// banks, for stores as well as for the operand reads.
struct StageMap {
  int key, part;
  bool v;
};

__device__ __forceinline__ StageMap stage_map(int t) {
  const int w = t >> 6, l = t & 63;
  StageMap m;
  if (l < 32) {
    const int gq = l >> 3;
    m = StageMap{8 * w + (l & 7), 2 * (gq & 1) + (gq >> 1), false};
  } else {
    const int l2 = l - 32, grp = l2 >> 3;
    m = StageMap{8 * w + ((l2 & 7) >> 1) + 4 * (grp & 1), 2 * (grp >> 1) + (l2 & 1), true};
  }
  return m;
}

// The thread's staged bytes start at this offset into cache row 0 (K or V).
__device__ __forceinline__ const uint8_t *stage_base(const StepArgs &a) {
  const StageMap m = stage_map(threadIdx.x);
  return (m.v ? a.v_cache : a.k_cache) + m.part * 32;
}

__device__ __forceinline__ void stage_load_row(const uint8_t *base, uint32_t row, StageIn &in) {
  const uint8_t *src = base + (uint64_t)row * ROW;
  in.x[0] = *reinterpret_cast<const uint4 *>(src);
  in.x[1] = *reinterpret_cast<const uint4 *>(src + 16);
}

// key0 + 63 < MAX_SPLIT_LDS: a piece holds at most MAX_SPLIT_LDS keys and the
// steps are clamped to the piece's last one.
__device__ __forceinline__ void stage_load(const uint8_t *base, const uint32_t *lrows, int key0,
                                           StageIn &in) {
  stage_load_row(base, (lrows + stage_map(threadIdx.x).key)[key0], in);
}

// Slot of chunk q of a V part: odd parts rotate by one.
__device__ __forceinline__ int v_slot(int part, int q) { return (q - (part & 1)) & 3; }

__device__ __forceinline__ void stage_store(const StageIn &in, Stage &st) {
  const StageMap m = stage_map(threadIdx.x);
  const f16x8 c[4] = {fp8x8_to_f16(in.x[0].x, in.x[0].y), fp8x8_to_f16(in.x[0].z, in.x[0].w),
                      fp8x8_to_f16(in.x[1].x, in.x[1].y), fp8x8_to_f16(in.x[1].z, in.x[1].w)};
  // per-lane offsets (no branch: K and V lanes share each store instruction)
  uint8_t *dst = m.v ? st.v + m.key * VROW + m.part * 64 : st.k + m.key * KROW;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int slot = m.v ? v_slot(m.part, q) : (4 * m.part + q) ^ (m.key & 15);
    *reinterpret_cast<f16x8 *>(dst + 16 * slot) = c[q];
  }
}

// A operand of S^T: key tile t of sub-chunk sc, K-step kk, KV head g.
__device__ __forceinline__ f16x8 k_operand(const Stage &st, int sc, int t, int kk, int n, int j,
                                           int g) {
  // chunk 8g + 4kk + j of key 32sc + 16t + n, at slot (8g + 4kk) ^ j ^ n
  return *reinterpret_cast<const f16x8 *>(st.k + (32 * sc + 16 * t + n) * KROW +
                                           16 * ((8 * g + 4 * kk) ^ j ^ n));
}

// A operand of O^T = V^T . P^T: dim tile dt of sub-chunk sc, KV head g.  Lane
// (n, j) receives dim 16dt + n of keys 4j..4j+3 (elements 0-3) and
// 16+4j..16+4j+3 (elements 4-7), the keys whose P it holds.
__device__ __forceinline__ f16x8 v_operand(const Stage &st, int sc, int dt, int n, int j, int g) {
  // dims 16dt + 4(n%4).. of head g: part 2g + dt/2, chunk 2(dt%2) + (n%4)/2, 8 B in
  const int part = 2 * g + (dt >> 1), q = 2 * (dt & 1) + ((n & 3) >> 1);
  const uint8_t *p = st.v + (32 * sc + 4 * j + (n >> 2)) * VROW + part * 64 + 16 * v_slot(part, q) +
                     8 * (n & 1);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * VROW));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8, v);
}

// Verify blocks stage the raw fp8 rows instead: a ring of VRING slots, each
// one step of 64 keys (8 KB of K rows, then 8 KB of V rows, 128 B per key),
// filled by the gfx950 direct global -> LDS loads (global_load_lds_dwordx4:
// lane l's 16 bytes land at the wave's LDS base + 16 l).  Wave w loads keys
// 8w..8w+7 of a step, 8 lanes per row; 16-byte chunk c of key x sits at slot
// c ^ vswz(x).  The operands are converted to fp16 (exactly) as they are
// read: K with ds_read_b64, V^T with the 8-bit transposing read
// ds_read_b64_tr_b8 (within a 16-lane group, lane 2k + h names 8 bytes of
// row k and lane i receives byte i of each of the 8 rows, probed on the GPU).
// vswz keeps both kinds of read on distinct banks in each 32-lane pass: a K
// read (16 keys of a tile, one chunk, both 8-byte halves) meets the 16
// distinct 16-byte bank groups 8 (x % 2) + (c ^ vswz(x)), and so does a V^T
// read (keys 4j..4j+3 and 16+4j..16+4j+3 for two adjacent j).  Half the LDS
// bytes of the fp16 stage move per step, and no registers or VALU work go
// into staging.
// Wait for this wave's vector memory operations down to v outstanding
// (vmcnt only; gfx9 encoding with expcnt and lgkmcnt at their maxima), and a
// barrier without a fence (the memory clobber keeps LDS accesses on their
// side of it).
#define VM_WAIT(v) \
  __builtin_amdgcn_s_waitcnt(((v) & 0xF) | (0x7 << 4) | (0xF << 8) | (((v) >> 4) << 14))
#define LDS_BARRIER() asm volatile("s_barrier" ::: "memory")
#ifndef MUSEATTN_VRING
#define MUSEATTN_VRING 3
#endif
constexpr int VRING = MUSEATTN_VRING;     // ring slots: VRING - 1 steps in flight
constexpr int VSLOT = STAGE_KEYS * ROW;   // bytes of one tensor's rows in a slot
static_assert(VRING >= 3 && VRING <= 4, "ring depth");

// Slot k of the ring: its own LDS object, so the compiler can tell the slot
// an LDS read touches from the slots the loads still in flight fill.
template <int K>
__device__ __forceinline__ uint8_t *vring_slot() {
  __shared__ __attribute__((aligned(1024))) uint8_t slot[2 * VSLOT];
  return slot;
}

__device__ __forceinline__ int vswz(int x) { return ((x >> 1) & 7) ^ (((x >> 4) & 1) << 2); }

// This thread's key of a step (wave w: keys 8w..8w+7, 8 lanes per key).
__device__ __forceinline__ int vkey(int tid) { return 8 * (tid >> 6) + ((tid & 63) >> 3); }

// The two direct loads (K row, V row) of this thread's 16 bytes of a step:
// key vkey(tid), its chunk (lane % 8) ^ vswz(key) from cache row `row`.
// AUX: the loads' cache-policy bits (2: non-temporal; each load instruction
// reads 8 whole rows, so no line is wanted again by a later one).
template <int AUX>
__device__ __forceinline__ void vring_issue(uint8_t *slot, const uint8_t *kc, const uint8_t *vc,
                                            uint32_t row, int tid) {
  const int c = (tid & 7) ^ vswz(vkey(tid));
  const uint64_t off = (uint64_t)row * ROW + 16 * c;
  uint8_t *dst = slot + 1024 * (tid >> 6);
  __builtin_amdgcn_global_load_lds((const void *)(kc + off), (__attribute__((address_space(3))) void *)dst,
                                   16, 0, AUX);
  __builtin_amdgcn_global_load_lds((const void *)(vc + off),
                                   (__attribute__((address_space(3))) void *)(dst + VSLOT), 16, 0, AUX);
}

// The operands of one sub-chunk from the fp8 ring, as 8 raw fp8 bytes each:
//  * kr[2t + kk], the A operand of S^T for key tile t and K-step kk of KV head
//    g: dims 32kk + 8j..+7 of key 32sc + 16t + n in lane (n, j);
//  * vr[dt], the A operand of O^T = V^T . P^T for dim tile dt: lane (n, j)
//    receives dim 16dt + n of keys 4j..4j+3 (bytes 0-3) and 16+4j..16+4j+3
//    (bytes 4-7); it names 8 bytes (dims 16dt + 8 (n % 2)..) of the
//    (n / 2)-th of those keys.
// The 8 reads are issued in one asm block that waits for them itself: the
// compiler would otherwise make every read of a slot wait for all the ring
// loads in flight, since it cannot tell the slots apart once their code is
// shared.  Every output is written only by the wait inside the block and
// none overlaps an address input (early clobber).
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
  return (uint32_t)(uintptr_t)(lds_u8 *)p;
}
__device__ __forceinline__ void ring_operands(const uint8_t *slot, int sc, int n, int j, int g,
                                              i32x2 (&kr)[4], i32x2 (&vr)[4]) {
  uint32_t ka[4], va[4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int x = 32 * sc + 16 * t + n, c = 4 * g + 2 * kk + (j >> 1);
      ka[2 * t + kk] = lds_addr(slot + x * ROW + 16 * (c ^ vswz(x)) + 8 * (j & 1));
    }
  const int k = n >> 1;
  const int xv = 32 * sc + (k < 4 ? 4 * j + k : 12 + 4 * j + k);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    va[dt] = lds_addr(slot + VSLOT + xv * ROW + 16 * ((4 * g + dt) ^ vswz(xv)) + 8 * (n & 1));
  asm volatile(
      "ds_read_b64 %0, %8\n\t"
      "ds_read_b64 %1, %9\n\t"
      "ds_read_b64 %2, %10\n\t"
      "ds_read_b64 %3, %11\n\t"
      "ds_read_b64_tr_b8 %4, %12\n\t"
      "ds_read_b64_tr_b8 %5, %13\n\t"
      "ds_read_b64_tr_b8 %6, %14\n\t"
      "ds_read_b64_tr_b8 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(vr[0]), "=&v"(vr[1]),
        "=&v"(vr[2]), "=&v"(vr[3])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3])
      : "memory");
}

// IEEE maximum (gfx950 v_maximum3_f32; no operand canonicalisation needed).
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Mask, online softmax and O^T += V^T . P^T for column tile c of one
// sub-chunk whose first key is u0.  s0, s1: the two key tiles of S^T, already
// relative to the reference max (the products start from -m), or raw while
// the column has no reference yet.
__device__ __forceinline__ void block_tile(f32x4 s0, f32x4 s1, const f16x8 (&va)[4], f16x8 ones,
                                           int u0, int j, BlockState &st, int c) {
  float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  if (st.scaled) {   // uniform; products of q * 2^-e back to log2 units
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[i] = ldexpf(sc[i], st.e[c]);
  }
  if (u0 < st.ulo[c] || u0 + CHUNK - 1 > st.uhi[c]) {   // uniform
    // score i is key u0 + 4j + off_i, off_i = 16 (i / 4) + i % 4
    const int elo = st.lo[c] - u0 - 4 * j, ehi = st.hi[c] - u0 - 4 * j;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = (i >> 2) * 16 + (i & 3);
      if (off < elo || off > ehi) sc[i] = -INFINITY;
    }
  }
  // four 3-input maxima
  const float m01 = fmax_ieee(fmax_ieee(sc[0], sc[1]), sc[2]);
  const float m23 = fmax_ieee(fmax_ieee(sc[3], sc[4]), sc[5]);
  const float lmax = fmax_ieee(fmax_ieee(sc[6], sc[7]), fmax_ieee(m01, m23));
  // Lazy reference max: it moves only when a score passes it by more than
  // RESCALE_SLACK (so P <= 2^SLACK), or for the column's first visible keys.
  if (__any(lmax > st.thr[c])) {
    const bool fresh = st.m[c] == -INFINITY;
    const float cm = head_max(lmax);   // the column's max, relative (or raw if fresh)
    float d, alpha;
    if (fresh) {
      d = cm == -INFINITY ? 0.0f : cm;
      alpha = 1.0f;
      st.m[c] = cm;
    } else {
      // only a column past the slack moves: the branch is taken for the whole
      // wave, and a column's numbers must not depend on its neighbours'
      d = cm > RESCALE_SLACK ? cm : 0.0f;
      alpha = __builtin_amdgcn_exp2f(-d);
      st.m[c] += d;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[i] -= d;
#pragma unroll
    for (int dt = 0; dt < 5; ++dt) st.o[dt][c] *= alpha;
    const float nm = st.m[c] == -INFINITY ? 0.0f : ldexpf(-st.m[c], -st.e[c]);
    st.negm[c] = f32x4{nm, nm, nm, nm};
    st.thr[c] = st.m[c] == -INFINITY ? -INFINITY : RESCALE_SLACK;
  }
  float pv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pv[i] = __builtin_amdgcn_exp2f(sc[i]);
  f16x8 ph;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f16x2 h = __builtin_convertvector((f32x2{pv[i], pv[i + 1]}), f16x2);
    ph[i] = h[0];
    ph[i + 1] = h[1];
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    st.o[dt][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[dt], ph, st.o[dt][c], 0, 0, 0);
  st.o[4][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, ph, st.o[4][c], 0, 0, 0);
}

// One sub-chunk (32 keys from u0) for the wave's nc live column tiles.
__device__ __forceinline__ void block_subchunk(const Stage &stg, int sc, int u0, int lane, int g,
                                               int nc, const f16x8 (&qf)[2][2], BlockState &st) {
  const int n = lane & 15, j = lane >> 4;
  f16x8 ka[2][2], va[4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ka[t][kk] = k_operand(stg, sc, t, kk, n, j, g);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) va[dt] = v_operand(stg, sc, dt, n, j, g);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c >= nc) break;   // uniform
    f32x4 s0 = st.negm[c], s1 = st.negm[c];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[0][kk], qf[c][kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[1][kk], qf[c][kk], s1, 0, 0, 0);
    }
    block_tile(s0, s1, va, st.ones, u0, j, st, c);
  }
}

// block_subchunk on a verify ring slot (fp8 rows, converted as read).
__device__ __forceinline__ void block_subchunk8(const uint8_t *slot, int sc, int u0, int lane,
                                                int g, int nc, const f16x8 (&qf)[2][2],
                                                BlockState &st) {
  const int n = lane & 15, j = lane >> 4;
  i32x2 kr[4], vr[4];
  ring_operands(slot, sc, n, j, g, kr, vr);
  f16x8 ka[2][2], va[4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      ka[t][kk] = fp8x8_to_f16((uint32_t)kr[2 * t + kk][0], (uint32_t)kr[2 * t + kk][1]);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) va[dt] = fp8x8_to_f16((uint32_t)vr[dt][0], (uint32_t)vr[dt][1]);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c >= nc) break;   // uniform
    f32x4 s0 = st.negm[c], s1 = st.negm[c];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[0][kk], qf[c][kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[1][kk], qf[c][kk], s1, 0, 0, 0);
    }
    block_tile(s0, s1, va, st.ones, u0, j, st, c);
  }
}

// Split and QK-norm of one (token, head) query and RoPE on sliding layers
// (task page "Gated attention decode", section "What to compute", first three
// lines of the listing).  Lane (n, j) holds dims 16j..16j+15: the head's
// rmsnorm is a sum over its 4 lanes (n, n+16, n+32, n+48), and the RoPE
// partner (dim +-32) sits in lane (n, j ^ 2) = lane ^ 32.  y = rmsnorm(q) *
// w_q * q_scale, rotated.  cs: the token's 32 (cos, sin) pairs in LDS.
struct QIn {
  uint4 r0, r1;   // the lane's 16 bf16 values of q
};

__device__ __forceinline__ QIn load_q_in(const StepArgs &a, int t, int head, int j) {
  const uint16_t *src = a.qkv + (size_t)t * QKV_W + head * D + 16 * j;
  return QIn{*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 8)};
}

__device__ __forceinline__ void q_values(const StepArgs &a, const QIn &in, const f32x4 (&wv)[4],
                                         int j, const float2 *cs, float (&y)[16]) {
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
  const float rden = 1.0f / sqrtf(ms + a.eps);   // q is not rounded to a code: one reciprocal
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] = x[k] * rden * wv[k >> 2][k & 3] * a.q_scale;
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
}

// One K-step of the B operand of S^T = K . Q^T: q[16j + 8 half + i] * mul
// (i < 8), split into bf16 hi + lo.
__device__ __forceinline__ void pack_q(const float (&y)[16], int half, float mul, bf16x8 &hi,
                                       bf16x8 &lo) {
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f32x2 f = {y[8 * half + i] * mul, y[8 * half + i + 1] * mul};
    const bf16x2 h = __builtin_convertvector(f, bf16x2);
    const bf16x2 l = __builtin_convertvector(f - __builtin_convertvector(h, f32x2), bf16x2);
    hi[i] = h[0]; hi[i + 1] = h[1];
    lo[i] = l[0]; lo[i + 1] = l[1];
  }
}

// Blocks: one K-step of the B operand of S^T in fp16, q[8j + i (+32)] * mul.
__device__ __forceinline__ f16x8 pack_q16(const float (&y)[16], int half, float mul) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f16x2 h = __builtin_convertvector((f32x2{y[8 * half + i] * mul, y[8 * half + i + 1] * mul}),
                                            f16x2);
    r[i] = h[0];
    r[i + 1] = h[1];
  }
  return r;
}

// Blocks: the power-of-two exponent e >= 0 that keeps a column's |q| * qmul *
// 2^-e below 2^15 (fp16 holds up to 65504); 0 for any ordinary input.
__device__ __forceinline__ int q_exponent(const float (&y)[16], float qmul) {
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(y[k] * qmul));
  amax = head_max(amax);
  if (!(amax >= 32768.0f) || amax == INFINITY) return 0;
  int ex;
  frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
  return ex - 15;
}

// Decode: head n's column of the block-diagonal Q^T.  K-step kk covers KV head
// kk/2, so it holds head n's values when n/8 == kk/2 and zeros otherwise; q is
// multiplied by log2(e)/8 and kv_scale (qmul).
__device__ __forceinline__ void make_q(const StepArgs &a, const QIn &in, const f32x4 (&wv)[4],
                                       int lane, float qmul, const float2 *cs, QOps &qo) {
  const int n = lane & 15, j = lane >> 4;
  float y[16];
  q_values(a, in, wv, j, cs, y);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8 hi, lo;
    pack_q(y, kk & 1, (n >> 3) == (kk >> 1) ? qmul : 0.0f, hi, lo);
    qo.op[kk][0][lane] = hi;
    qo.op[kk][1][lane] = lo;
  }
}

// The new k and v rows of the block tokens flagged in `own` (bit jt = token
// jt of request b, at position pos[jt]): k = rmsnorm(k) * w_k, rotated on
// sliding layers, then fp8(k / kv_scale) and fp8(v / kv_scale) into cache row
// row(b, p) (task page "Gated attention decode", section "What to compute",
// the cache line of the listing).  Wave 0/1: k head 0/1, wave 2/3: v head 0/1;
// lane = dim.  All tokens' inputs are loaded before any is used.
template <int NT>   // block tokens: 1 (decode) or up to 8 (verify)
struct RowIn {
  uint32_t x[NT];   // the lane's k or v value of each block token (bf16 bits)
  float wk;
};

template <int NT>
__device__ __forceinline__ RowIn<NT> load_row_in(const StepArgs &a, int b) {
  const int wave = threadIdx.x >> 6, d = threadIdx.x & 63;
  const int off = (wave < 2 ? K_OFF : V_OFF) + (wave & 1) * D + d;
  RowIn<NT> in;
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    const int t = b * a.L + (jt < a.L ? jt : a.L - 1);
    in.x[jt] = a.qkv[(size_t)t * QKV_W + off];
  }
  in.wk = a.wk[d];
  return in;
}

template <int NT>
__device__ __forceinline__ void write_new_rows(const StepArgs &a, int b, unsigned own,
                                               const int (&pos)[NT], const float2 (*cs)[32],
                                               const RowIn<NT> &in) {
  const int wave = threadIdx.x >> 6, d = threadIdx.x & 63;
  const bool is_k = wave < 2;
  const int g = wave & 1;
  const float wk = in.wk;
  float x[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) x[jt] = bf16_bits_to_f32((uint16_t)in.x[jt]);
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
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

// Every round is loaded and stored, with indices clamped into the key range
// (rounds past the piece's chunks repeat its last entry): the loads carry no
// branch, so the compiler can count them exactly and a later wait for an
// earlier load need not wait for these.  The table row is a uniform base and
// the entry a 32-bit offset from it.
__device__ __forceinline__ void load_table_in(const StepArgs &a, int b, const KeyRange &r,
                                              int kstart, TableIn &in) {
  const int tid = threadIdx.x;
  const int shift = a.page_size == 1 ? 0 : 6;
  const int32_t *trow = a.table + (int64_t)b * a.table_stride;
#pragma unroll
  for (int it = 0; it < MAX_SPLIT_LDS / THREADS; ++it) {
    const int v = kstart + tid + it * THREADS;
    in.u[it] = v < r.klo ? r.klo : (v > r.khi ? r.khi : v);
    in.unit[it] = trow[in.u[it] >> shift];
  }
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

template <int MODE>
struct Lds {
  static constexpr int MAXU = MODE == 3 ? MAX_UNITS : MAX_BATCH;   // plan units
  static constexpr int NCS = MODE == 3 ? PREFILL_TB : 8;           // tokens per unit
  uint32_t lrows[MAX_SPLIT_LDS];
  float2 cs[NCS][32];        // RoPE (cos, sin) per token of the unit and pair
  float rinv[32];            // RoPE inverse frequency per pair (sliding layers)
  union {
    float sm_o[WAVES][HQ][D];   // decode: the 8 waves' O per head
    float mrg[2][64][68];       // verify merge: chunk lane 1's O per KV head and column (padded)
    Stage stg[MODE == 3 ? 2 : 1];   // prefill: the K/V stage buffers (verify: a ring of its own)
  };
  float mrg_ml[2][64][2];       // verify merge: its (max, sum) per column
  QOps dq;                      // decode: the token's Q^T operands
  float sm_m[WAVES][HQ];
  float sm_l[WAVES][HQ];
  int pref[MAXU + 1];
  int scan[WAVES];           // the plan's per-wave totals
  int req_len[MAXU];         // end of each unit's key range (last token's position + 1)
  int req_p0[MAXU];          // position of each unit's first token (sliding layers)
};

// One decode segment: chunks [x, y) of request b's key range (chunk i = keys
// kbase + 32i ..), processed by the whole work-group, leaving one partial per
// head in slot `slot`.  The 8 waves take interleaved chunks and both KV heads.
template <int NBUF, bool NTV, bool NTP>
__device__ __forceinline__ void process_segment(const StepArgs &a, int b, const KeyRange &r,
                                                int p_tok, int x, int y, int slot, Lds<0> &sh,
                                                bool first, bool second) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const float qmul = a.kv_scale * (LOG2E / 8.0f);
  const int nseg = y - x;
  const int npieces = (nseg + PIECE_CHUNKS - 1) / PIECE_CHUNKS;
  auto piece_x = [&](int pc) { return x + (int)div_floor((int64_t)pc * nseg, npieces); };

  // One batch of loads for everything the segment starts with: the first
  // piece's table entries, the token's q row and norm weights and the inputs
  // of its new k/v row (kept as raw bits: converting them here would wait for
  // the loads).  The token's position came with the plan (p_tok).
  TableIn tin;
  load_table_in(a, b, r, r.kbase + x * CHUNK, tin);
  // every wave loads q (wave 0 builds the Q^T operands) and the new row's
  // inputs (waves 0-3 write it): no branch around the loads
  const QIn qin = load_q_in(a, b, n, j);   // head n of the token
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(a.wq + 16 * j);
  const f32x4 wv[4] = {w4[0], w4[1], w4[2], w4[3]};
  const RowIn<1> rin = load_row_in<1>(a, b);   // every wave: no branch around the loads
  int pt = p_tok < 0 ? 0 : (p_tok > a.max_seq_len - 1 ? a.max_seq_len - 1 : p_tok);
  const int pos[1] = {pt};   // decode: one block token, token b
  __builtin_amdgcn_sched_barrier(0);
  stamp(a, TS_ISSUED, first);
  // the token's RoPE (cos, sin) pairs (L = 1), computed while the loads fly
  float2 csv = make_float2(1.0f, 0.0f);
  if (a.sliding && tid < 32) csv = rope_cs_inv(pos[0], sh.rinv[tid]);

  __syncthreads();   // the previous segment is done with sh.cs, sh.lrows and the merge buffers
  if (a.sliding) {
    if (tid < 32) sh.cs[0][tid] = csv;
    __syncthreads();
  }
  store_table(a, tin, sh.lrows);
  stamp(a, TS_TABLE, first);

  // per-token key ranges: the causal bound is the token's position p, the
  // window (sliding layers) starts 2047 keys before it
  auto token_range = [&](bool live, int p, int &lo, int &hi) {
    hi = live ? (p < r.khi ? p : r.khi) : -1;
    lo = a.sliding ? p - (WINDOW - 1) : 0;
  };
  TokState ts;
  token_range(true, pos[0], ts.lo, ts.hi);
  ts.m = -INFINITY;
  ts.l = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) ts.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave == 0) make_q(a, qin, wv, lane, qmul, sh.cs[0], sh.dq);   // published by the barrier below
  // New rows of the block tokens whose key falls in this segment: only this
  // work-group reads them, so a workgroup release before the barrier orders
  // the writes before its own loads.
  const int pn = pos[0];
  const unsigned owned = pn >= r.klo && pn <= r.khi && (pn - r.kbase) / CHUNK >= x &&
                         (pn - r.kbase) / CHUNK < y;
  if (owned && wave < 4) write_new_rows<1>(a, b, owned, pos, sh.cs, rin);
  stamp(a, TS_QREADY, first);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  stamp(a, TS_SETUP, first);
  stamp(a, TS_SEG2_SETUP, second);

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
    const int c0 = wave;
    const int cstep = WAVES;
    const int nloc = nchunks > c0 ? (nchunks - c0 + cstep - 1) / cstep : 0;
    if (nloc > 0) {
      const int last = nloc - 1;
      auto rows_of = [&](int i) { return sh.lrows + (c0 + i * cstep) * CHUNK; };
      auto key_of = [&](int i) { return kstart + (c0 + i * cstep) * CHUNK; };
      RowBuf buf[NBUF];
#pragma unroll
      for (int k = 0; k < NBUF; ++k)
        load_rows<NTV>(buf[k], a.k_cache, a.v_cache, rows_of(k < last ? k : last), n, j);
      int i = 0;
      for (; i + NBUF <= nloc; i += NBUF) {
#pragma unroll
        for (int k = 0; k < NBUF; ++k) {
          compute_chunk(buf[k], key_of(i + k), lane, ts, sh.dq);
          const int inext = i + k + NBUF;
          load_rows<NTV>(buf[k], a.k_cache, a.v_cache, rows_of(inext < last ? inext : last), n, j);
        }
      }
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k)
        if (i + k < nloc) compute_chunk(buf[k], key_of(i + k), lane, ts, sh.dq);
    }
  }

  stamp(a, TS_STREAM, first);
  // Lane (n, j) holds O^T of head n at V-row bytes 8(4j + r) + mt, r < 4: KV
  // head j/2, dims 32(j%2) + 8r + mt.  Only lanes whose KV head is head n's
  // own hold meaningful values.
  const bool own = (j >> 1) == (n >> 3);
  const int dbase = 32 * (j & 1);
  const float lsum = head_sum(ts.l);
  if (j == 0) {
    sh.sm_m[wave][n] = ts.m;
    sh.sm_l[wave][n] = lsum;
  }
  if (own) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float *dst = &sh.sm_o[wave][n][dbase + 8 * rr];
      *reinterpret_cast<f32x4 *>(dst) =
          f32x4{ts.o[0][rr], ts.o[1][rr], ts.o[2][rr], ts.o[3][rr]};
      *reinterpret_cast<f32x4 *>(dst + 4) =
          f32x4{ts.o[4][rr], ts.o[5][rr], ts.o[6][rr], ts.o[7][rr]};
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
  part_store<NTP>(reinterpret_cast<f32x2 *>(a.part_o + e * D + d2), o);
  if ((tid & 31) == 0) {
    part_store<NTP>(reinterpret_cast<f32x2 *>(a.part_ml + e * 2), f32x2{M, lt});
  }
  stamp(a, TS_PARTIAL, first);
}

// Blocks: the q of one (token, head) column in the lane layout of the block
// path -- lane (n, j) holds dims 8j..8j+7 (K-step 0) and 32+8j..32+8j+7
// (K-step 1) -- normed over the head's 4 lanes and, on sliding layers,
// rotated (each RoPE pair (i, i+32) sits in one lane); cs: the token's 32
// (cos, sin) pairs in LDS.
struct QIn2 {
  uint4 lo, hi;   // bf16 dims 8j..8j+7 and 32+8j..32+8j+7
};

__device__ __forceinline__ QIn2 load_q_in2(const StepArgs &a, int t, int head, int j) {
  const uint16_t *src = a.qkv + (size_t)t * QKV_W + head * D + 8 * j;
  return QIn2{*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 32)};
}

__device__ __forceinline__ void q_values2(const StepArgs &a, const QIn2 &in, const f32x4 (&wv)[4],
                                          int j, const float2 *cs, float (&y)[16]) {
  const uint32_t raw[8] = {in.lo.x, in.lo.y, in.lo.z, in.lo.w, in.hi.x, in.hi.y, in.hi.z, in.hi.w};
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
  const float rden = 1.0f / sqrtf(ms + a.eps);   // q is not rounded to a code: one reciprocal
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] = x[k] * rden * wv[k >> 2][k & 3] * a.q_scale;
  if (a.sliding) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // pair 8j + i: x_i c - x_{i+32} s, x_{i+32} c + x_i s
      const float2 c = cs[8 * j + i];
      const float lo = y[i], hi = y[8 + i];
      y[i] = lo * c.x - hi * c.y;
      y[8 + i] = hi * c.x + lo * c.y;
    }
  }
}

#ifndef MUSEATTN_BLOCK_PREFETCH
#define MUSEATTN_BLOCK_PREFETCH 2
#endif

// One segment of a verify (MODE 2) or prefill (MODE 3) block: chunks [x, y)
// of unit (b, blk)'s key range, leaving one partial per (token, head) in slot
// `slot`.
template <int MODE, bool NTP = false, bool NTV = false>
__device__ __forceinline__ void process_segment_block(const StepArgs &a, int b, int blk,
                                                      const KeyRange &r, int x, int y, int slot,
                                                      Lds<MODE> &sh, bool first, bool second) {
  constexpr bool VERIFY = MODE == 2;
  constexpr int NR = MUSEATTN_BLOCK_PREFETCH;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const float qmul = a.kv_scale * (LOG2E / 8.0f);
  const int nseg = y - x;
  const int npieces = (nseg + PIECE_CHUNKS - 1) / PIECE_CHUNKS;
  auto piece_x = [&](int pc) { return x + (int)div_floor((int64_t)pc * nseg, npieces); };
  const int g = wave & 1;
  const int cq = VERIFY ? (wave >> 1) & 1 : wave >> 1;   // column tiles 2cq, 2cq + 1
  const int cl = VERIFY ? wave >> 2 : 0;                 // verify: the wave's sub-chunk
  const int j0 = blk * a.tb;                             // the unit's first block token
  const int nt = a.L - j0 < a.tb ? a.L - j0 : a.tb;      // tokens in the unit
  int nc = (nt + 1) / 2 - 2 * cq;                        // the wave's live column tiles
  nc = nc < 0 ? 0 : (nc > 2 ? 2 : nc);
  auto tok = [&](int c) { return 4 * cq + 2 * c + (n >> 3); };   // unit token of the lane column

  // One batch of loads.  First what the first steps' stage loads depend on:
  // (verify) the block tokens' positions, lane j holding token j % 8's (a
  // per-lane value: kept in a vector register, it is not waited for until
  // used), and the table entries of the rows this thread stages in the first
  // BLOCK_PREFETCH steps.  Then the first piece's table entries, the column
  // tokens' positions and q, the RoPE position of this thread's pair, the q
  // norm weights and (verify) the new rows' inputs.  No load sits behind a
  // branch, so the compiler counts them exactly: a wait for the first ones is
  // not a wait for the batch.
  const int shift = a.page_size == 1 ? 0 : 6;
  const int nsteps0 = (piece_x(1) - x + 1) >> 1;
  const int cs_tk = tid >> 5;   // sliding: this thread's RoPE pair is (token cs_tk, pair tid % 32)
  int posv = 0;
  if constexpr (VERIFY) posv = a.positions[b * a.L + ((lane & 7) < a.L ? (lane & 7) : a.L - 1)];
  constexpr int NE = VERIFY ? VRING - 1 : NR;   // steps whose loads may leave early
  const int ekey = VERIFY ? vkey(tid) : stage_map(tid).key;
  int eu[NE], eunit[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int v = r.kbase + x * CHUNK + (k < nsteps0 ? k : nsteps0 - 1) * STAGE_KEYS + ekey;
    eu[k] = v < r.klo ? r.klo : (v > r.khi ? r.khi : v);
    eunit[k] = a.table[(int64_t)b * a.table_stride + (eu[k] >> shift)];
  }
  TableIn tin;
  load_table_in(a, b, r, r.kbase + x * CHUNK, tin);
  int cpos[2];
  QIn2 qin[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int tk = tok(c);
    const int t = b * a.L + j0 + (tk < nt ? tk : nt - 1);
    cpos[c] = a.positions[t];
    qin[c] = load_q_in2(a, t, 8 * g + (n & 7), j);
  }
  const int cs_p = a.positions[b * a.L + j0 + (cs_tk < nt ? cs_tk : nt - 1)];
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(a.wq);
  const f32x4 wv[4] = {w4[2 * j], w4[2 * j + 1], w4[8 + 2 * j], w4[8 + 2 * j + 1]};
  RowIn<8> rin;
  if constexpr (VERIFY) rin = load_row_in<8>(a, b);
  __builtin_amdgcn_sched_barrier(0);

  // Verify: the block tokens whose new rows fall in this segment (only this
  // work-group reads them; they are written below): lane j < 8 tests token j.
  unsigned owned = 0;
  int pos[8];
  if constexpr (VERIFY) {
    const int jt = lane & 7;
    const bool in = lane < 8 && jt < a.L && posv >= r.klo && posv <= r.khi &&
                    (posv - r.kbase) / CHUNK >= x && (posv - r.kbase) / CHUNK < y;
    owned = (unsigned)__ballot(in);
#pragma unroll
    for (int t2 = 0; t2 < 8; ++t2) pos[t2] = __builtin_amdgcn_readlane(posv, t2);
  }
  // The first steps' stage loads leave now, from the thread's own table
  // entries, so they overlap the set-up below -- unless the segment holds new
  // rows, which must be written first, or (verify) another segment of this
  // work-group may still be reading the ring slots they fill.
  const bool early = owned == 0 && (!VERIFY || first);
  const uint8_t *sbase = stage_base(a);
  StageIn in[NR];
  uint4 ek0, ev0, ek1, ev1, ek2, ev2;   // verify: the first steps' rows, this thread's 16 B
  if (early) {
    const uint32_t units = (uint32_t)(a.num_rows >> shift);
    uint32_t row[NE];
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      uint32_t un = (uint32_t)eunit[k];
      un = un < units ? un : units - 1;
      row[k] = (un << shift) + (uint32_t)(eu[k] & (a.page_size - 1));
    }
    if constexpr (VERIFY) {
      // into registers: a direct load into LDS would be waited for at the
      // set-up's first LDS access; the bytes go to their ring slots before
      // the set-up barrier
      const int c = (tid & 7) ^ vswz(ekey);
      const uint8_t *k0 = a.k_cache + (uint64_t)row[0] * ROW + 16 * c;
      const uint8_t *v0 = a.v_cache + (uint64_t)row[0] * ROW + 16 * c;
      const uint8_t *k1 = a.k_cache + (uint64_t)row[1] * ROW + 16 * c;
      const uint8_t *v1 = a.v_cache + (uint64_t)row[1] * ROW + 16 * c;
      ek0 = *reinterpret_cast<const uint4 *>(k0);
      ev0 = *reinterpret_cast<const uint4 *>(v0);
      ek1 = *reinterpret_cast<const uint4 *>(k1);
      ev1 = *reinterpret_cast<const uint4 *>(v1);
      if constexpr (VRING > 3) {
        ek2 = *reinterpret_cast<const uint4 *>(a.k_cache + (uint64_t)row[2] * ROW + 16 * c);
        ev2 = *reinterpret_cast<const uint4 *>(a.v_cache + (uint64_t)row[2] * ROW + 16 * c);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NE; ++k) stage_load_row(sbase, row[k], in[k]);
    }
  }

  stamp(a, TS_ISSUED, first);
  // RoPE (cos, sin) of the unit's tokens (512 threads: up to 16 tokens x 32
  // pairs), computed while the loads fly
  float2 csv = make_float2(1.0f, 0.0f);
  if (a.sliding && cs_tk < nt) csv = rope_cs_inv(cs_p, sh.rinv[tid & 31]);

  __syncthreads();   // the previous segment is done with sh.cs, sh.lrows and the stage buffers
  if (a.sliding) {
    if (cs_tk < nt) sh.cs[cs_tk][tid & 31] = csv;
    __syncthreads();
  }
  store_table(a, tin, sh.lrows);
  stamp(a, TS_TABLE, first);

  f16x8 qf[2][2];
  BlockState st;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int tk = tok(c);
    float yq[16];
    q_values2(a, qin[c], wv, j, sh.cs[tk < nt ? tk : nt - 1], yq);
    st.e[c] = q_exponent(yq, qmul);
    const float mul = ldexpf(qmul, -st.e[c]);
    qf[c][0] = pack_q16(yq, 0, mul);
    qf[c][1] = pack_q16(yq, 1, mul);
    // causal bound: the token's position; window: 2047 keys before it
    const int p = cpos[c];
    st.hi[c] = tk < nt ? (p < r.khi ? p : r.khi) : -1;
    st.lo[c] = a.sliding ? p - (WINDOW - 1) : 0;
    // The columns' common visible range.  A tile's columns belong to two
    // tokens, held by lanes 0 and 8; a dead token (its results are never
    // written) does not narrow it.
    {
      const int lo0 = __builtin_amdgcn_readlane(st.lo[c], 0), lo1 = __builtin_amdgcn_readlane(st.lo[c], 8);
      const int hi0 = __builtin_amdgcn_readlane(st.hi[c], 0), hi1 = __builtin_amdgcn_readlane(st.hi[c], 8);
      const bool live1 = tok(c) - (n >> 3) + 1 < nt;   // uniform: the tile's second token
      st.ulo[c] = live1 ? (lo0 > lo1 ? lo0 : lo1) : lo0;
      st.uhi[c] = live1 ? (hi0 < hi1 ? hi0 : hi1) : hi0;
    }
    st.thr[c] = -INFINITY;
    st.m[c] = -INFINITY;
    st.negm[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 5; ++dt) st.o[dt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  st.scaled = __any(st.e[0] != 0 || st.e[1] != 0);
  {
    // made opaque to the compiler, so that it keeps the operand in registers
    // instead of rebuilding it with moves at every tile
    uint32_t w[4] = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};   // fp16 1.0 pairs
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(w[i]));
    st.ones = __builtin_bit_cast(f16x8, w);
  }
  if constexpr (VERIFY) {
    // the new rows: a workgroup release before the barrier orders the writes
    // before this work-group's own loads.  (Prefill rows come from rows_kernel.)
    if (owned && wave < 4) write_new_rows<8>(a, b, owned, pos, sh.cs, rin);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (early) {   // the first steps' rows into their ring slots
      const int o = 1024 * wave + 16 * lane;
      *reinterpret_cast<uint4 *>(vring_slot<0>() + o) = ek0;
      *reinterpret_cast<uint4 *>(vring_slot<0>() + VSLOT + o) = ev0;
      *reinterpret_cast<uint4 *>(vring_slot<1>() + o) = ek1;
      *reinterpret_cast<uint4 *>(vring_slot<1>() + VSLOT + o) = ev1;
      if constexpr (VRING > 3) {
        *reinterpret_cast<uint4 *>(vring_slot<2>() + o) = ek2;
        *reinterpret_cast<uint4 *>(vring_slot<2>() + VSLOT + o) = ev2;
      }
    }
  }
  stamp(a, TS_QREADY, first);
  __syncthreads();   // the row ids (and verify's new rows) are in place
  stamp(a, TS_SETUP, first);
  stamp(a, TS_SEG2_SETUP, second);

  for (int pc = 0; pc < npieces; ++pc) {
    const int px = piece_x(pc), py = piece_x(pc + 1);
    const int nch = py - px;
    const int kstart = __builtin_amdgcn_readfirstlane(r.kbase + px * CHUNK);   // uniform
    if (pc > 0) {
      __syncthreads();   // every wave is done with the previous rows
      TableIn tn;
      load_table_in(a, b, r, kstart, tn);
      __builtin_amdgcn_sched_barrier(0);
      store_table(a, tn, sh.lrows);
      __syncthreads();
    }
    // Steps of two sub-chunks (64 keys).
    const int nsteps = (nch + 1) >> 1;
    if constexpr (VERIFY) {
      // The fp8 ring: step t fills slot t % VRING, VRING - 1 steps ahead.  At
      // step t a wave waits for its own loads of t (the 2 (VRING - 2) of the
      // later steps may stay in flight), the barrier makes everyone's visible
      // and frees slot (t - 1) % VRING, which then takes step t + VRING - 1.
      // Steps past the piece's end load its last step again (cache hits), so
      // every wave issues the same loads and the counts hold.  The barrier is
      // a bare s_barrier: a fence would also wait for the later steps' loads.
      auto issue_step = [&](uint8_t *sl, int t) {
        const int sk = (t < nsteps ? t : nsteps - 1) * STAGE_KEYS + vkey(tid);
        vring_issue<NTV ? 2 : 0>(sl, a.k_cache, a.v_cache, sh.lrows[sk], tid);
      };
      if (pc > 0 || !early) {   // uniform
        issue_step(vring_slot<0>(), 0);
        issue_step(vring_slot<1>(), 1);
        if constexpr (VRING > 3) issue_step(vring_slot<2>(), 2);
      }
      // one step: slot RD holds it, slot WR takes step t + VRING - 1 (each
      // slot named at compile time, so the compiler sees that the loads in
      // flight fill other slots than the one read)
      auto step = [&](auto rd_tag, auto wr_tag, int t) {
        VM_WAIT(2 * (VRING - 2));
        LDS_BARRIER();
        issue_step(vring_slot<decltype(wr_tag)::value>(), t + VRING - 1);
        if (2 * t + cl < nch && nc > 0)
          block_subchunk8(vring_slot<decltype(rd_tag)::value>(), cl, kstart + (2 * t + cl) * CHUNK,
                          lane, g, nc, qf, st);
      };
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      using S3 = std::integral_constant<int, (VRING > 3 ? 3 : 2)>;
      for (int s0 = 0; s0 < nsteps; s0 += VRING) {   // the branches are uniform
        if constexpr (VRING == 3) {
          step(S0{}, S2{}, s0);
          if (s0 + 1 < nsteps) step(S1{}, S0{}, s0 + 1);
          if (s0 + 2 < nsteps) step(S2{}, S1{}, s0 + 2);
        } else {
          step(S0{}, S3{}, s0);
          if (s0 + 1 < nsteps) step(S1{}, S0{}, s0 + 1);
          if (s0 + 2 < nsteps) step(S2{}, S1{}, s0 + 2);
          if (s0 + 3 < nsteps) step(S3{}, S2{}, s0 + 3);
        }
      }
      VM_WAIT(0);   // the loads past the piece's end are in before the slots are reused
    } else {
      // The stage loads of step s go to register set s % NR, issued NR steps
      // ahead; in the steady state they are unconditional (steps past the end
      // are clamped to the last), so the compiler counts them and waits only
      // for the set it stores next.
      auto step_key = [&](int s) { return (s < nsteps ? s : nsteps - 1) * STAGE_KEYS; };
      auto compute = [&](int s) {
        const Stage &sg = sh.stg[s & 1];
        if (nc > 0) {
          block_subchunk(sg, 0, kstart + 2 * s * CHUNK, lane, g, nc, qf, st);
          if (2 * s + 1 < nch)
            block_subchunk(sg, 1, kstart + (2 * s + 1) * CHUNK, lane, g, nc, qf, st);
        }
      };
      if (pc > 0 || !early) {   // uniform
#pragma unroll
        for (int k = 0; k < NR; ++k) stage_load(sbase, sh.lrows, step_key(k), in[k]);
      }
      stage_store(in[0], sh.stg[0]);
      stage_load(sbase, sh.lrows, step_key(NR), in[0]);
      __syncthreads();
      int s = 0;
      for (; s + NR < nsteps; s += NR) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          compute(s + k);
          stage_store(in[(k + 1) % NR], sh.stg[(s + k + 1) & 1]);
          stage_load(sbase, sh.lrows, step_key(s + k + 1 + NR), in[(k + 1) % NR]);
          __syncthreads();
        }
      }
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        if (s + k < nsteps) {   // uniform
          compute(s + k);
          if (s + k + 1 < nsteps) stage_store(in[(k + 1) % NR], sh.stg[(s + k + 1) & 1]);
          __syncthreads();
        }
      }
    }
  }

  stamp(a, TS_STREAM, first);
  float lsum[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) lsum[c] = st.o[4][c][0];
  if constexpr (VERIFY) {
    // Merge sub-chunk lane 1 into lane 0 (a one-chunk segment leaves lane 1
    // empty).  The merge buffers share LDS with the stage buffers, which every
    // wave has finished with at the last step's barrier.
    if (nseg > 1) {   // uniform
      if (cl == 1) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c >= nc) break;
          const int col = 16 * (2 * cq + c) + n;
          float *row = sh.mrg[g][col];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4 *>(row + 16 * dt + 4 * j) = st.o[dt][c];
          if (j == 0) {
            sh.mrg_ml[g][col][0] = st.m[c];
            sh.mrg_ml[g][col][1] = lsum[c];
          }
        }
      }
      __syncthreads();
      if (cl == 0) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c >= nc) break;
          const int col = 16 * (2 * cq + c) + n;
          const float *row = sh.mrg[g][col];
          const float m1 = sh.mrg_ml[g][col][0], l1 = sh.mrg_ml[g][col][1];
          const float M = fmaxf(st.m[c], m1);
          const float c0 = st.m[c] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st.m[c] - M);
          const float c1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
          lsum[c] = lsum[c] * c0 + l1 * c1;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            st.o[dt][c] = st.o[dt][c] * c0 + *reinterpret_cast<const f32x4 *>(row + 16 * dt + 4 * j) * c1;
          st.m[c] = M;
        }
      }
    }
  }
  if (cl == 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int tk = tok(c);
      if (c >= nc) break;
      if (tk >= nt) continue;
      const size_t e = ((size_t)slot * a.tb + tk) * HQ + 8 * g + (n & 7);
      if (j == 0) {
        part_store<NTP>(reinterpret_cast<f32x2 *>(a.part_ml + e * 2), f32x2{st.m[c], lsum[c]});
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        part_store<NTP>(reinterpret_cast<f32x4 *>(a.part_o + e * D + 16 * dt + 4 * j), st.o[dt][c]);
    }
  }
  stamp(a, TS_PARTIAL, first);
}

// The attention kernel.  Every work-group derives the same plan from the
// device-side sequence lengths: plan unit u (a request, or one token group of
// a request when L > 8) spans chunks [pref[u], pref[u+1]) of the concatenated
// chunk space, and work-group w takes an equal contiguous share of it
// (counting each unit start as seg_cost chunks), so no work-group idles while
// another still has a long split.  A share that crosses unit boundaries is
// processed one segment per unit; segment (w, u) writes its partial to slot
// w + u (slots are unique because both w and u grow along the chunk space).
// The combine kernel then merges each unit's slots.  NTV and NTP: rows read
// (decode: V; verify: K and V into the ring) and partials stored
// non-temporally, chosen by launch_attn from the step's size.
template <int MODE, int NBUF, bool NTV = false, bool NTP = false>
__global__ __launch_bounds__(THREADS, 2) void attn_kernel(StepArgs a) {
  __shared__ __attribute__((aligned(16))) Lds<MODE> sh;
  constexpr int MAXU = Lds<MODE>::MAXU;
  const int tid = threadIdx.x;
  stamp(a, TS_ENTRY);
  const int NU = a.nunits;

  // chunk-count prefix sums over the plan units (RPT per thread)
  constexpr int RPT = MAXU / THREADS;
  int cnt[RPT], sum = 0;
  {
    // lengths (and, on sliding layers, first positions) of the thread's
    // units, loaded as one batch
    int sl[RPT], p0[RPT], ublk[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int u = RPT * tid + k < NU ? RPT * tid + k : NU - 1;
      int ub;
      unit_of(a, u, ub, ublk[k]);
      sl[k] = a.seq_lens[ub];
      p0[k] = a.positions[ub * a.L + ublk[k] * a.tb];   // (decode reads its token's here)
    }
    __builtin_amdgcn_sched_barrier(0);
    // the RoPE frequencies (kernel arguments), read while the lengths are in
    // flight; the segments take them from LDS, with no load of their own
    if (a.sliding && tid < 32) sh.rinv[tid] = rope_inv(tid);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int len = unit_len(a, sl[k], ublk[k]);
      cnt[k] = RPT * tid + k < NU ? request_chunks(range_from(a, len, p0[k])) : 0;
      sum += cnt[k];
      sh.req_len[RPT * tid + k] = len;
      sh.req_p0[RPT * tid + k] = p0[k];
    }
  }
  {
    // exclusive prefix sum over the threads: a shuffle scan inside each wave,
    // then the 8 wave totals through LDS
    const int lane = tid & 63, wave = tid >> 6;
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      incl += lane >= off ? v : 0;
    }
    if (lane == 63) sh.scan[wave] = incl;
    __syncthreads();
    int run = incl - sum, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2) {
      const int t = sh.scan[w2];
      run += w2 < wave ? t : 0;
      total += t;
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int u = RPT * tid + k;
      if (u < NU) sh.pref[u] = run;
      run += cnt[k];
    }
    if (tid == 0) sh.pref[NU] = total;
  }
  __syncthreads();
  stamp(a, TS_PLAN);
  // Cost space: unit u occupies seg_cost units (its segment start-up, in
  // chunk-equivalents), then its chunks, then end_cost units (the new rows
  // the holder of its last chunk writes), so unit u starts at cost Q_u =
  // pref[u] + u * (seg_cost + end_cost).  Work-groups take equal cost
  // shares; one whose share covers a unit's start or end gets
  // correspondingly fewer chunks.
  const int pen = a.seg_cost, per = a.seg_cost + a.end_cost;
  const int64_t Ct = (int64_t)sh.pref[NU] + (int64_t)NU * per;
  const int w = blockIdx.x;
  const int G = Ct < a.work_groups ? (int)Ct : a.work_groups;
  if (w == 0) {
    // the plan, for the combine kernel: chunk prefix sums and work-groups used
    for (int i = tid; i <= NU; i += THREADS) a.plan[i] = sh.pref[i];
    if (tid == 0) a.plan[NU + 1] = G;
  }
  if (w >= G) {   // uniform over the work-group
    stamp_count(a, TS_SEGMENTS, 0);
    stamp(a, TS_EXIT);
    return;
  }
  const int64_t cb = div_floor((int64_t)w * Ct, G), ce = div_floor((int64_t)(w + 1) * Ct, G);
  auto cost_of = [&](int uu) { return (int64_t)sh.pref[uu] + (int64_t)uu * per; };
  int u = 0;
  {
    int hi = NU - 1;
    while (u < hi) {   // largest u whose cost range starts at or before cb
      const int mid = (u + hi + 1) >> 1;
      if (cost_of(mid) <= cb) u = mid; else hi = mid - 1;
    }
  }
  int nsegs = 0;
  for (; u < NU && cost_of(u) < ce; ++u) {
    const int64_t q0 = cost_of(u) + pen;            // cost of chunk 0 of unit u
    const int64_t nb = sh.pref[u + 1] - sh.pref[u];
    const int64_t xs = cb - q0, ys = ce - q0;
    const int x = (int)(xs > 0 ? xs : 0);
    const int y = (int)(ys < nb ? ys : nb);
    if (y <= x) continue;
    const KeyRange r = range_from(a, sh.req_len[u], sh.req_p0[u]);
    int b, blk;
    unit_of(a, u, b, blk);
    stamp(a, TS_SEG2_START, nsegs == 1);
    if constexpr (MODE == 0)
      process_segment<NBUF, NTV, NTP>(a, b, r, sh.req_p0[u], x, y, w + u, sh, nsegs == 0,
                                 nsegs == 1);
    else
      process_segment_block<MODE, NTP, NTV>(a, b, blk, r, x, y, w + u, sh, nsegs == 0,
                                            nsegs == 1);
    ++nsegs;
  }
  stamp_count(a, TS_SEGMENTS, (uint64_t)nsegs);
  stamp(a, TS_EXIT);
}

// Decode steps whose rows may exceed this many bytes (B x the keys a request
// may see x 256 B) read V by non-temporal loads and store their partials
// non-temporally; verify steps read K and V into their ring non-temporally
// (verify B 32, L 8: step 161.6 -> 156.4 us; at B 16, 410 MB, no gain).  Measured on decode B 32, contexts U[60K, 100K] (672 MB per
// step, 2.6x the 256 MB Infinity Cache): attention kernel 125 -> 115 us, at
// pools of 1.5 to 80 GB.  At B 16 (about 340 MB per step) part of a step's
// rows is still cached at the next step, and the ordinary loads were faster
// (61.0 vs 62.0 us).
#ifndef MUSEATTN_NT_MIN_STEP_BYTES
#define MUSEATTN_NT_MIN_STEP_BYTES (512ll << 20)
#endif
// With 64-row pages the switch comes earlier: decode B 16, contexts U[60K,
// 100K], page size 64 (331 MB per step): attention kernel 59.5 -> 58.0 us,
// where at page size 1 (337 MB) the ordinary loads stay ahead (61.3 vs 61.8).
#ifndef MUSEATTN_NT_MIN_STEP_BYTES_P64
#define MUSEATTN_NT_MIN_STEP_BYTES_P64 (256ll << 20)
#endif
// Verify blocks store their partials (8 tokens' worth per slot) non-temporally
// from this many bytes of rows per step: verify L 8 over 80K keys 22.6 ->
// 22.3 us per step, B 32 full 161.8 -> 158.7, B 32 sliding 23.2 -> 22.5; a
// sliding block of one request (0.5 MB) was slower with them (16.3 vs 16.8).
#ifndef MUSEATTN_NTP_MIN_VERIFY_BYTES
#define MUSEATTN_NTP_MIN_VERIFY_BYTES (4ll << 20)
#endif

void launch_attn(const StepArgs &a, hipStream_t stream) {
  const dim3 grid(a.work_groups), block(THREADS);
  const long long keys = a.sliding && a.max_seq_len > WINDOW ? WINDOW : a.max_seq_len;
  const long long step_bytes = (long long)a.B * keys * 2 * ROW;
  const long long nt_min = a.page_size == 64 ? MUSEATTN_NT_MIN_STEP_BYTES_P64 : MUSEATTN_NT_MIN_STEP_BYTES;
  if (a.L == 1 && step_bytes > MUSEATTN_NT_MIN_STEP_BYTES)
    hipLaunchKernelGGL((attn_kernel<0, MUSEATTN_DECODE_NBUF, true, true>), grid, block, 0, stream, a);
  else if (a.L == 1 && step_bytes > nt_min)
    hipLaunchKernelGGL((attn_kernel<0, MUSEATTN_DECODE_NBUF, true>), grid, block, 0, stream, a);
  else if (a.L == 1)
    hipLaunchKernelGGL((attn_kernel<0, MUSEATTN_DECODE_NBUF>), grid, block, 0, stream, a);
  else if (a.L <= 8 && step_bytes > MUSEATTN_NT_MIN_STEP_BYTES)
    hipLaunchKernelGGL((attn_kernel<2, 1, true, true>), grid, block, 0, stream, a);
  else if (a.L <= 8 && step_bytes > MUSEATTN_NTP_MIN_VERIFY_BYTES)
    hipLaunchKernelGGL((attn_kernel<2, 1, false, true>), grid, block, 0, stream, a);
  else if (a.L <= 8)
    hipLaunchKernelGGL((attn_kernel<2, 1>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_kernel<3, 1>), grid, block, 0, stream, a);
}

}  // namespace museattn

