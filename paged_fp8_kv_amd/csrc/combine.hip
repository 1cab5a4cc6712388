// Merge of the key-axis partials and the gated output norm: for token t and
// head h, a = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) * kv_scale over the
// slots of t's request, then out = rmsnorm(a) * w_o * sigmoid(gate) in bf16
// (task page "Gated attention decode", section "What to compute", last line
// of the listing; output shape from the same section).
//
// Decode and verify blocks (many slots per token): one 256-thread work-group
// per (token, head).  The plan entries, the gate and the output-norm weight
// are loaded as one batch; then 16 slot lanes x 16 dimension quads each merge
// their slots online (running max, rescaled sum and output), so the partials
// take a single memory round trip; LDS merges the 16 slot lanes and one wave
// finishes the gated norm.
//
// Prefill blocks (thousands of tokens, a few slots each): one work-group per
// token, 16 lanes per head, each lane merging all slots for 4 dimensions.
#include "device_common.h"
#include "launch.h"

namespace museattn {

// KB > 0: each slot lane loads its first KB slots in one batch (for units with
// many slots: one long request spread over every work-group).  SPEC (one
// request, B = 1): the request's slots are work-groups 0 .. G - 1, so the
// loads of slots sl, sl + 16, .., below nspec go out with the plan's instead
// of after it (one memory round trip instead of two); the plan then selects
// [s0, s1] among them, and slots from s = 16 KB on, if any, follow the plan.
template <int KB, bool SPEC = false>
__global__ __launch_bounds__(256) void combine_kernel(StepArgs a, int nspec) {
  __shared__ float sm_m[16], sm_l[16];
  __shared__ __attribute__((aligned(16))) float sm_o[16][D];

  stamp_combine(a, 0);
  const int th = blockIdx.x;          // t * 16 + h
  const int t = th / HQ, h = th % HQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // token t = block token jl of request b, token jt of plan unit u
  const int b = t / a.L, jl = t % a.L;
  const int blk = jl / a.tb, jt = jl - blk * a.tb;
  const int u = b * a.nblk + blk, NU = a.nunits;
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml);
  const f32x4 *po = reinterpret_cast<const f32x4 *>(a.part_o);
  auto entry = [&](int s) { return ((size_t)s * a.tb + jt) * HQ + h; };
  const int sl = tid >> 4, dq = tid & 15;
  int64_t p0, p1, pn;
  int G;
  float2 sv[SPEC ? KB : 1];
  f32x4 sx[SPEC ? KB : 1];
  if constexpr (SPEC) {
    // vector loads (an atomic load is never a scalar one), so that the slot
    // loads behind them are not held up by a wait for the plan
    auto ldv = [](const int *p) {
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    };
    p0 = ldv(a.plan + u);
    p1 = ldv(a.plan + u + 1);
    pn = ldv(a.plan + NU);
    G = ldv(a.plan + NU + 1);
    // every candidate slot, clamped into [0, nspec): no branch, so no wait
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int sk = sl + 16 * k < nspec ? sl + 16 * k : nspec - 1;
      const size_t e = entry(sk);
      sv[k] = ml[e];
      sx[k] = po[e * (D / 4) + dq];
    }
  } else {
    p0 = a.plan[u];
    p1 = a.plan[u + 1];
    pn = a.plan[NU];
    G = a.plan[NU + 1];
  }
  const int64_t Ct = pn + (int64_t)NU * (a.seg_cost + a.end_cost);
  const float g = bf16_bits_to_f32(a.qkv[(size_t)t * QKV_W + G_OFF + h * D + lane]);
  const float wo = a.wo[lane];
  // slots of unit u: w + u for the work-groups w whose cost share meets its
  // chunks (chunk c of unit u sits at cost p0 + u (seg_cost + end_cost) +
  // seg_cost + c)
  int s0 = 0, s1 = -1;
  if (p1 > p0) {
    const int64_t q0 = p0 + (int64_t)u * (a.seg_cost + a.end_cost) + a.seg_cost;
    s0 = wg_of_chunk(q0, Ct, G) + u;
    s1 = wg_of_chunk(q0 + (p1 - p0) - 1, Ct, G) + u;
  }

  // online merge of slots s0 + sl, s0 + sl + 16, ... (four loads in flight)
  float m = -INFINITY, l = 0.0f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  auto merge = [&](float2 v, f32x4 x) {
    const float mn = fmaxf(m, v.x);
    const float c0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    const float c1 = v.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(v.x - mn);
    l = l * c0 + v.y * c1;
    o = o * c0 + x * c1;
    m = mn;
  };
  int s = s0 + sl;
  if constexpr (SPEC) {
    // only this step's slots of the unit count (the others may hold anything)
    bool keep[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int sk = sl + 16 * k;
      keep[k] = sk >= s0 && sk <= s1 && sk < nspec && sv[k].x != -INFINITY;
      if (keep[k]) m = fmaxf(m, sv[k].x);
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      if (keep[k]) {
        const float c = __builtin_amdgcn_exp2f(sv[k].x - m);
        l += sv[k].y * c;
        o += sx[k] * c;
      }
    }
    s = sl;   // the lane's first slot the batch did not cover
    while (s < nspec || s < s0) s += 16;
  } else if constexpr (KB > 0) {
    float2 v[KB];
    f32x4 x[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int sk = s + 16 * k;
      v[k] = float2{-INFINITY, 0.0f};
      x[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (sk <= s1) {
        const size_t e = entry(sk);
        v[k] = ml[e];
        x[k] = po[e * (D / 4) + dq];
      }
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) m = fmaxf(m, v[k].x);
    if (m != -INFINITY) {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const float c = v[k].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(v[k].x - m);
        l += v[k].y * c;
        o += x[k] * c;
      }
    }
    s += 16 * KB;
  }
  for (; s + 48 <= s1; s += 64) {
    float2 v[4];
    f32x4 x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t e = entry(s + 16 * k);
      v[k] = ml[e];
      x[k] = po[e * (D / 4) + dq];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) merge(v[k], x[k]);
  }
  for (; s <= s1; s += 16) {
    const size_t e = entry(s);
    merge(ml[e], po[e * (D / 4) + dq]);
  }
  *reinterpret_cast<f32x4 *>(&sm_o[sl][4 * dq]) = o;
  if (dq == 0) {
    sm_m[sl] = m;
    sm_l[sl] = l;
  }
  __syncthreads();

  if (wave == 0) {
    const int d = lane;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) M = fmaxf(M, sm_m[k]);
    float od = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float c = sm_m[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sm_m[k] - M);
        od += c * sm_o[k][d];
        lsum += c * sm_l[k];
      }
    }
    const float av = lsum > 0.0f ? od / lsum * a.kv_scale : 0.0f;
    const float ms2 = wave_sum(av * av) * (1.0f / 64.0f);
    const float y = av / sqrtf(ms2 + a.eps) * wo;
    a.out[(size_t)t * (HQ * D) + h * D + d] = f32_to_bf16_bits(y / (1.0f + expf(-g)));
  }
  stamp_combine(a, 1);
}

// Prefill merge: work-group t = token t; lane group hg = lane / 16 of wave w
// takes head h = 4w + hg, lane dq = lane % 16 its dims 4dq..4dq+3.  All heads
// of a token share its unit's slots.
__global__ __launch_bounds__(256) void combine_tokens_kernel(StepArgs a) {
  stamp_combine(a, 0);
  const int t = blockIdx.x;
  const int tid = threadIdx.x, h = tid >> 4, dq = tid & 15;
  const int b = t / a.L, jl = t % a.L;
  const int blk = jl / a.tb, jt = jl - blk * a.tb;
  const int u = b * a.nblk + blk, NU = a.nunits;
  const int64_t p0 = a.plan[u], p1 = a.plan[u + 1];
  const int G = a.plan[NU + 1];
  const int64_t Ct = (int64_t)a.plan[NU] + (int64_t)NU * (a.seg_cost + a.end_cost);
  const uint2 graw = *reinterpret_cast<const uint2 *>(a.qkv + (size_t)t * QKV_W + G_OFF + h * D +
                                                      4 * dq);
  const f32x4 wo = *reinterpret_cast<const f32x4 *>(a.wo + 4 * dq);
  int s0 = 0, s1 = -1;
  if (p1 > p0) {
    const int64_t q0 = p0 + (int64_t)u * (a.seg_cost + a.end_cost) + a.seg_cost;
    s0 = wg_of_chunk(q0, Ct, G) + u;
    s1 = wg_of_chunk(q0 + (p1 - p0) - 1, Ct, G) + u;
  }
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml);
  const f32x4 *po = reinterpret_cast<const f32x4 *>(a.part_o);
  auto entry = [&](int s) { return ((size_t)s * a.tb + jt) * HQ + h; };

  float m = -INFINITY, l = 0.0f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  auto merge = [&](float2 v, f32x4 x) {
    const float mn = fmaxf(m, v.x);
    const float c0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    const float c1 = v.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(v.x - mn);
    l = l * c0 + v.y * c1;
    o = o * c0 + x * c1;
    m = mn;
  };
  int s = s0;
  for (; s + 3 <= s1; s += 4) {
    float2 v[4];
    f32x4 x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t e = entry(s + k);
      v[k] = ml[e];
      x[k] = po[e * (D / 4) + dq];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) merge(v[k], x[k]);
  }
  for (; s <= s1; ++s) {
    const size_t e = entry(s);
    merge(ml[e], po[e * (D / 4) + dq]);
  }
  const f32x4 av = l > 0.0f ? o * (a.kv_scale / l) : f32x4{0.f, 0.f, 0.f, 0.f};
  const float ms2 = row16_sum(av[0] * av[0] + av[1] * av[1] + av[2] * av[2] + av[3] * av[3]) *
                    (1.0f / 64.0f);
  const float rn = 1.0f / sqrtf(ms2 + a.eps);
  const uint32_t gw[2] = {graw.x, graw.y};
  uint32_t packed[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float g0 = __uint_as_float(gw[k] << 16), g1 = __uint_as_float(gw[k] & 0xffff0000u);
    const float y0 = av[2 * k] * rn * wo[2 * k] / (1.0f + expf(-g0));
    const float y1 = av[2 * k + 1] * rn * wo[2 * k + 1] / (1.0f + expf(-g1));
    packed[k] = (uint32_t)f32_to_bf16_bits(y0) | ((uint32_t)f32_to_bf16_bits(y1) << 16);
  }
  *reinterpret_cast<uint2 *>(a.out + (size_t)t * (HQ * D) + h * D + 4 * dq) =
      uint2{packed[0], packed[1]};
  stamp_combine(a, 1);
}

#ifndef MUSEATTN_TOKENS_COMBINE_MIN_B
#define MUSEATTN_TOKENS_COMBINE_MIN_B 24
#endif
#ifndef MUSEATTN_COMBINE_BATCH_SLOTS
#define MUSEATTN_COMBINE_BATCH_SLOTS 48
#endif
// Most candidate slots a one-request merge loads with its plan (at most 3 per
// slot lane).  With more, a work-group's partials are tens of KB, the merge is
// bound by the bytes per CU rather than by round trips, and the unconditional
// loads cost more than the round trip saves (graph-timed steps: 256 slots, 3f
// 23.0 vs 22.0 us; 79, c1 11.6 vs 11.3; 31, c0 9.8 vs 10.5).
#ifndef MUSEATTN_COMBINE_SPEC_SLOTS
#define MUSEATTN_COMBINE_SPEC_SLOTS 48
#endif
static_assert(MUSEATTN_COMBINE_SPEC_SLOTS <= 48, "3 candidate slots per slot lane at most");
#ifndef MUSEATTN_TOKENS_COMBINE_MIN_L
#define MUSEATTN_TOKENS_COMBINE_MIN_L 2
#endif

void launch_combine(const StepArgs &a, hipStream_t stream) {
  if (a.L > 8 || (a.L >= MUSEATTN_TOKENS_COMBINE_MIN_L && a.B >= MUSEATTN_TOKENS_COMBINE_MIN_B)) {
    hipLaunchKernelGGL(combine_tokens_kernel, dim3(a.B * a.L), dim3(256), 0, stream, a);
    return;
  }
  // one request over many work-groups leaves many slots per unit: at most
  // one per work-group, and no more than its chunks (plus start-up) allow
  int64_t keys = a.max_seq_len;
  if (a.sliding) keys = keys < WINDOW + a.L - 1 ? keys : WINDOW + a.L - 1;
  const int64_t chunks = (keys + CHUNK - 1) / CHUNK + 1 + a.seg_cost + a.end_cost;
  const int64_t slots = a.B == 1 ? (chunks < a.work_groups ? chunks : a.work_groups)
                                 : a.work_groups / a.B + 2;
  const dim3 grid(a.B * a.L * HQ);
  if (a.B == 1 && slots <= MUSEATTN_COMBINE_SPEC_SLOTS) {
    // one request: its slots are work-groups 0 .. G - 1, G at most its cost
    // (chunks, one more for a window's alignment, start-up and end costs)
    const int nspec = (int)slots;
    if (nspec <= 16)
      hipLaunchKernelGGL((combine_kernel<1, true>), grid, dim3(256), 0, stream, a, nspec);
    else
      hipLaunchKernelGGL((combine_kernel<3, true>), grid, dim3(256), 0, stream, a, nspec);
  } else if (slots > MUSEATTN_COMBINE_BATCH_SLOTS) {
    hipLaunchKernelGGL((combine_kernel<16>), grid, dim3(256), 0, stream, a, 0);
  } else {
    hipLaunchKernelGGL((combine_kernel<0>), grid, dim3(256), 0, stream, a, 0);
  }
}

}  // namespace museattn
