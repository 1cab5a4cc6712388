// Host side of libmuseattn: argument validation, the launch shape (a function
// of host shapes only, so a call can be captured into a HIP graph), workspace
// layout and the two launches.  See include/museattn.h for the contract.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/museattn.h"
#include "device_common.h"
#include "launch.h"

namespace museattn {
namespace {

constexpr int MAX_WORK_GROUPS = 65535;
constexpr int MAX_SEQ = 1 << 30;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Attention work-groups.  Each takes an equal share of all requests' key
// chunks; one 8-wave work-group per CU of MI355X (256 CUs) keeps every CU
// busy to the end without a tail.
int choose_work_groups(int L, int requested) {
  (void)L;
  if (requested > 0) return requested;
  return 256;
}

struct Layout {
  int work_groups;
  size_t plan_off, ml_off, o_off, ts_off, total;
};

// Plan units: up to 8 block tokens a request is one unit; beyond (prefill)
// its tokens form groups of PREFILL_TB.
int unit_tokens(int L) { return L <= 8 ? L : PREFILL_TB; }
int units_per_request(int L) { return (L + unit_tokens(L) - 1) / unit_tokens(L); }

Layout layout(int B, int L, int work_groups) {
  Layout ly;
  ly.work_groups = work_groups;
  const size_t units = (size_t)B * units_per_request(L);
  const size_t slots = (size_t)work_groups + units;   // partial slots w + u
  const size_t tb = unit_tokens(L);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  ly.plan_off = 0;
  ly.ml_off = ly.plan_off + al((units + 2) * sizeof(int));
  ly.o_off = ly.ml_off + al(slots * tb * HQ * 2 * sizeof(float));
  ly.ts_off = ly.o_off + al(slots * tb * HQ * D * sizeof(float));
  ly.total = ly.ts_off;
#ifdef MUSEATTN_PHASE_TIMES
  // the timestamps at the end: TS_SLOTS per attention work-group, then two
  // per combine work-group (at most one per token and head)
  ly.total += al(((size_t)work_groups * TS_SLOTS + 2 * (size_t)B * L * HQ) * sizeof(uint64_t));
#endif
  return ly;
}

// A segment start-up (batch of loads + first rows) is worth about this many
// 32-key chunks of one work-group's streaming (measured on MI355X).
#ifndef MUSEATTN_SEG_COST_VERIFY
#define MUSEATTN_SEG_COST_VERIFY 16
#endif
#ifndef MUSEATTN_SEG_COST_PREFILL
#define MUSEATTN_SEG_COST_PREFILL 16
#endif
#ifndef MUSEATTN_SEG_COST_DECODE
#define MUSEATTN_SEG_COST_DECODE 14
#endif
// The work-group holding a unit's last chunk also writes its new rows
// (prefill rows are written by their own kernel).
#ifndef MUSEATTN_END_COST_DECODE
#define MUSEATTN_END_COST_DECODE 0
#endif
#ifndef MUSEATTN_END_COST_VERIFY
#define MUSEATTN_END_COST_VERIFY 8
#endif
constexpr int MAX_COST = 64;
static_assert(MUSEATTN_SEG_COST_VERIFY <= MAX_COST && MUSEATTN_SEG_COST_PREFILL <= MAX_COST &&
                  MUSEATTN_SEG_COST_DECODE <= MAX_COST && MUSEATTN_END_COST_DECODE <= MAX_COST &&
                  MUSEATTN_END_COST_VERIFY <= MAX_COST,
              "plan costs are bounded for the 32-bit prefix sums");

int seg_cost(int L) {
  return L == 1 ? MUSEATTN_SEG_COST_DECODE
                : (L <= 8 ? MUSEATTN_SEG_COST_VERIFY : MUSEATTN_SEG_COST_PREFILL);
}
int end_cost(int L) {
  return L == 1 ? MUSEATTN_END_COST_DECODE : (L <= 8 ? MUSEATTN_END_COST_VERIFY : 0);
}

// Chunk-equivalents of the plan's cost space that one unit can occupy at
// most: its key range in 32-key chunks (one more for the alignment of a
// sliding window's start) plus the start-up and end costs.
int64_t max_unit_cost(int L, int max_seq_len, int layer_kind) {
  int64_t keys = max_seq_len;
  if (layer_kind == MUSEATTN_SLIDING) {
    const int64_t win = (int64_t)WINDOW + unit_tokens(L) - 1;
    keys = keys < win ? keys : win;
  }
  return (keys + CHUNK - 1) / CHUNK + 1 + 2 * MAX_COST;
}

int check_shapes(int B, int L, int max_seq_len, int page_size, int layer_kind,
                 const museattn_params *params) {
  if (page_size != 1 && page_size != 64) return MUSEATTN_ERR_PAGE_SIZE;
  if (layer_kind != MUSEATTN_FULL && layer_kind != MUSEATTN_SLIDING) return MUSEATTN_ERR_LAYER_KIND;
  if (B < 1 || B > MAX_BATCH || L < 1 || L > MAX_L || max_seq_len < L || max_seq_len > MAX_SEQ)
    return MUSEATTN_ERR_SHAPE;
  const int64_t units = (int64_t)B * units_per_request(L);
  if (units > MAX_UNITS) return MUSEATTN_ERR_SHAPE;
  // the kernels keep the plan's chunk prefix sums in 32-bit integers
  if (units * max_unit_cost(L, max_seq_len, layer_kind) >= (int64_t(1) << 31))
    return MUSEATTN_ERR_SHAPE;
  if (params == nullptr) return MUSEATTN_ERR_NULL;
  if (params->work_groups < 0 || params->work_groups > MAX_WORK_GROUPS) return MUSEATTN_ERR_PARAM;
  return MUSEATTN_OK;
}

// Host-side validation of a step's arguments (touches no device memory).
// has_ws: the caller passes the workspace (else the library's static scratch
// serves, and only its size is checked, by the caller of this function).
int check_step_args(const void *qkv, const int32_t *positions, const int32_t *table,
                    const int32_t *seq_lens, const void *k_cache, const void *v_cache,
                    float kv_scale, int page_size, int layer_kind, const void *out, int B, int L,
                    int table_stride, int max_seq_len, int64_t num_rows,
                    const museattn_params *params, bool has_ws, const void *workspace,
                    size_t workspace_bytes) {
  if (!qkv || !positions || !table || !seq_lens || !k_cache || !v_cache || !out || !params ||
      (has_ws && !workspace))
    return MUSEATTN_ERR_NULL;
  if (!params->q_norm_w || !params->k_norm_w || !params->o_norm_w) return MUSEATTN_ERR_NULL;
  const int st = check_shapes(B, L, max_seq_len, page_size, layer_kind, params);
  if (st != MUSEATTN_OK) return st;
  // rows are addressed as 32-bit indices on the device
  if (num_rows < page_size || num_rows % page_size != 0 || num_rows >= (int64_t(1) << 32))
    return MUSEATTN_ERR_SHAPE;
  if ((int64_t)table_stride * page_size < max_seq_len || table_stride < 1) return MUSEATTN_ERR_TABLE;
  // the kernels read q, k, v and gate slices of 16 B, the norm weights as
  // float4 and write 8-byte output pieces
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(qkv, 16) || !aligned(out, 8) ||
      !aligned(positions, 4) || !aligned(table, 4) || !aligned(seq_lens, 4) ||
      !aligned(params->q_norm_w, 16) || !aligned(params->k_norm_w, 16) ||
      !aligned(params->o_norm_w, 16))
    return MUSEATTN_ERR_ALIGN;
  if (!(std::isfinite(kv_scale) && kv_scale > 0.0f) ||
      !(std::isfinite(params->eps) && params->eps >= 0.0f) || !std::isfinite(params->q_scale) ||
      !(std::isfinite(params->rope_base) && params->rope_base > 0.0f))
    return MUSEATTN_ERR_PARAM;
  if (has_ws && (!aligned(workspace, 256) ||
                 workspace_bytes < layout(B, L, choose_work_groups(L, params->work_groups)).total))
    return MUSEATTN_ERR_WORKSPACE;
  // the buffers the step writes (out, the caches' new rows, the workspace)
  // must not overlap each other or anything the step reads: every work-group
  // re-reads seq_lens, positions and the table while others write
  struct Span {
    uintptr_t lo, hi;
  };
  auto span = [](const void *p, uint64_t bytes) {
    return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
  };
  auto meet = [](Span x, Span y) { return x.lo < y.hi && y.lo < x.hi; };
  const uint64_t T = (uint64_t)B * L;
  const Span written[4] = {span(out, T * HQ * D * 2), span(k_cache, (uint64_t)num_rows * ROW),
                           span(v_cache, (uint64_t)num_rows * ROW),
                           span(has_ws ? workspace : nullptr, has_ws ? workspace_bytes : 0)};
  const Span read[7] = {span(qkv, T * QKV_W * 2), span(positions, T * 4),
                        span(table, (uint64_t)B * table_stride * 4), span(seq_lens, (uint64_t)B * 4),
                        span(params->q_norm_w, D * 4), span(params->k_norm_w, D * 4),
                        span(params->o_norm_w, D * 4)};
  for (int i = 0; i < 4; ++i) {
    for (int k = i + 1; k < 4; ++k)
      if (meet(written[i], written[k])) return MUSEATTN_ERR_ALIAS;
    for (const Span &r : read)
      if (meet(written[i], r)) return MUSEATTN_ERR_ALIAS;
  }
  return MUSEATTN_OK;
}

// Enqueues one validated step: the kernels read and write `ws` as the
// workspace of museattn_workspace_bytes(...) bytes.
int enqueue_step(const void *qkv, const int32_t *positions, const int32_t *table,
                 const int32_t *seq_lens, void *k_cache, void *v_cache, float kv_scale,
                 int page_size, int layer_kind, void *out, void *stream, int B, int L,
                 int table_stride, int max_seq_len, int64_t num_rows,
                 const museattn_params *params, void *workspace, void *attn_start_event,
                 void *attn_end_event) {
  const Layout ly = layout(B, L, choose_work_groups(L, params->work_groups));
  char *ws = static_cast<char *>(workspace);

  StepArgs a;
  a.qkv = static_cast<const uint16_t *>(qkv);
  a.positions = positions;
  a.table = table;
  a.seq_lens = seq_lens;
  a.k_cache = static_cast<uint8_t *>(k_cache);
  a.v_cache = static_cast<uint8_t *>(v_cache);
  a.out = static_cast<uint16_t *>(out);
  a.wq = params->q_norm_w;
  a.wk = params->k_norm_w;
  a.wo = params->o_norm_w;
  a.plan = reinterpret_cast<int *>(ws + ly.plan_off);
  a.part_ml = reinterpret_cast<float *>(ws + ly.ml_off);
  a.part_o = reinterpret_cast<float *>(ws + ly.o_off);
  a.num_rows = num_rows;
  a.kv_scale = kv_scale;
  a.eps = params->eps;
  a.q_scale = params->q_scale;
  // RoPE inverse frequencies, one per pair: constants of the rotation (they
  // depend on rope_base only), rounded to fp32 as the angle product uses them
  for (int i = 0; i < 32; ++i)
    a.rope_inv[i] = (float)std::pow((double)params->rope_base, -(double)i / 32.0);
  a.B = B;
  a.L = L;
  a.table_stride = table_stride;
  a.max_seq_len = max_seq_len;
  a.page_size = page_size;
  a.sliding = layer_kind == MUSEATTN_SLIDING;
  a.work_groups = ly.work_groups;
  a.seg_cost = seg_cost(L);
  a.end_cost = end_cost(L);
  a.tb = unit_tokens(L);
  a.nblk = units_per_request(L);
  a.nunits = B * a.nblk;
#ifdef MUSEATTN_PHASE_TIMES
  a.ts = reinterpret_cast<uint64_t *>(ws + ly.ts_off);
#else
  a.ts = nullptr;
#endif

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();   // clear an error left by earlier, unrelated calls
  if (L > 8) launch_rows(a, s);   // prefill: every new row before any attention
  if (attn_start_event) (void)hipEventRecord(static_cast<hipEvent_t>(attn_start_event), s);
  launch_attn(a, s);
  if (attn_end_event) (void)hipEventRecord(static_cast<hipEvent_t>(attn_end_event), s);
  launch_combine(a, s);
  return hipGetLastError() == hipSuccess ? MUSEATTN_OK : MUSEATTN_ERR_LAUNCH;
}

// The step's scratch for callers that cannot allocate device memory
// (museattn_attn_step_noalloc): one fixed array per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: the kernels receive the address hipGetSymbolAddress returns
// for the current device, looked up once per device and kept here (the only
// state the library keeps between calls; it allocates nothing).
constexpr int MAX_DEVICES = 64;
static __device__ __align__(256) uint8_t scratch[MUSEATTN_STATIC_SCRATCH_BYTES];
std::atomic<uintptr_t> scratch_addr[MAX_DEVICES];   // 0 until looked up

// The device address of `scratch` on the device `stream` runs on (with that
// device current during the lookup); MUSEATTN_ERR_LAUNCH if HIP cannot say.
int scratch_for(hipStream_t stream, void **out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return MUSEATTN_ERR_LAUNCH;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return MUSEATTN_ERR_LAUNCH;
  if (dev < 0 || dev >= MAX_DEVICES) return MUSEATTN_ERR_LAUNCH;
  uintptr_t p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p == 0) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MUSEATTN_ERR_LAUNCH;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr || !aligned(ptr, 256)) return MUSEATTN_ERR_LAUNCH;
    p = (uintptr_t)ptr;
    scratch_addr[dev].store(p, std::memory_order_release);   // a racing lookup stores the same
  }
  *out = reinterpret_cast<void *>(p);
  return MUSEATTN_OK;
}

}  // namespace
}  // namespace museattn

using namespace museattn;

extern "C" {

int museattn_abi_version(void) { return MUSEATTN_ABI_VERSION; }

const char *museattn_strerror(int status) {
  switch (status) {
    case MUSEATTN_OK: return "ok";
    case MUSEATTN_ERR_NULL: return "a required pointer is null";
    case MUSEATTN_ERR_PAGE_SIZE: return "page_size must be 1 or 64";
    case MUSEATTN_ERR_LAYER_KIND: return "layer_kind must be MUSEATTN_FULL or MUSEATTN_SLIDING";
    case MUSEATTN_ERR_SHAPE:
      return "B, L, B * ceil(L / 16) (L > 8), max_seq_len, the plan's chunk count or num_rows "
             "out of range";
    case MUSEATTN_ERR_TABLE: return "table_stride < ceil(max_seq_len / page_size)";
    case MUSEATTN_ERR_ALIGN: return "misaligned pointer (caches, qkv and weights need 16 bytes, out 8)";
    case MUSEATTN_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case MUSEATTN_ERR_PARAM: return "kv_scale, eps, q_scale, rope_base or work_groups out of range";
    case MUSEATTN_ERR_ALIAS:
      return "a written buffer (out, k_cache, v_cache, workspace) overlaps another buffer";
    case MUSEATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int museattn_work_groups(int B, int L, int max_seq_len, int layer_kind, const museattn_params *params) {
  if (check_shapes(B, L, max_seq_len, 1, layer_kind, params) != MUSEATTN_OK) return 0;
  return choose_work_groups(L, params->work_groups);
}

size_t museattn_workspace_bytes(int B, int L, int max_seq_len, int page_size, int layer_kind,
                                const museattn_params *params) {
  if (check_shapes(B, L, max_seq_len, page_size, layer_kind, params) != MUSEATTN_OK) return 0;
  return layout(B, L, choose_work_groups(L, params->work_groups)).total;
}

int museattn_check_args(const void *qkv, const int32_t *positions, const int32_t *table,
                        const int32_t *seq_lens, const void *k_cache, const void *v_cache,
                        float kv_scale, int page_size, int layer_kind, const void *out, int B,
                        int L, int table_stride, int max_seq_len, int64_t num_rows,
                        const museattn_params *params, const void *workspace,
                        size_t workspace_bytes) {
  return check_step_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
                         layer_kind, out, B, L, table_stride, max_seq_len, num_rows, params, true,
                         workspace, workspace_bytes);
}

int museattn_attn_step_profiled(const void *qkv, const int32_t *positions, const int32_t *table,
                                const int32_t *seq_lens, void *k_cache, void *v_cache,
                                float kv_scale, int page_size, int layer_kind, void *out,
                                void *stream, int B, int L, int table_stride, int max_seq_len,
                                int64_t num_rows, const museattn_params *params, void *workspace,
                                size_t workspace_bytes, void *attn_start_event,
                                void *attn_end_event) {
  const int st = museattn_check_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale,
                                     page_size, layer_kind, out, B, L, table_stride, max_seq_len,
                                     num_rows, params, workspace, workspace_bytes);
  if (st != MUSEATTN_OK) return st;
  return enqueue_step(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
                      layer_kind, out, stream, B, L, table_stride, max_seq_len, num_rows, params,
                      workspace, attn_start_event, attn_end_event);
}

int museattn_attn_step(const void *qkv, const int32_t *positions, const int32_t *table,
                       const int32_t *seq_lens, void *k_cache, void *v_cache, float kv_scale,
                       int page_size, int layer_kind, void *out, void *stream, int B, int L,
                       int table_stride, int max_seq_len, int64_t num_rows,
                       const museattn_params *params, void *workspace, size_t workspace_bytes) {
  return museattn_attn_step_profiled(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale,
                                     page_size, layer_kind, out, stream, B, L, table_stride,
                                     max_seq_len, num_rows, params, workspace, workspace_bytes,
                                     nullptr, nullptr);
}

int museattn_attn_step_noalloc(const void *qkv, const int32_t *positions, const int32_t *table,
                               const int32_t *seq_lens, void *k_cache, void *v_cache,
                               float kv_scale, int page_size, int layer_kind, void *out,
                               void *stream, int B, int L, int table_stride, int max_seq_len,
                               int64_t num_rows, const museattn_params *params) {
  const int st = check_step_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale,
                                 page_size, layer_kind, out, B, L, table_stride, max_seq_len,
                                 num_rows, params, false, nullptr, 0);
  if (st != MUSEATTN_OK) return st;
  if (layout(B, L, choose_work_groups(L, params->work_groups)).total > MUSEATTN_STATIC_SCRATCH_BYTES)
    return MUSEATTN_ERR_WORKSPACE;
  void *ws = nullptr;
  const int sst = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (sst != MUSEATTN_OK) return sst;
  // Nothing in the scratch has to start at zero: the attention kernel writes
  // the plan and every partial slot the combine kernel reads.
  return enqueue_step(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
                      layer_kind, out, stream, B, L, table_stride, max_seq_len, num_rows, params,
                      ws, nullptr, nullptr);
}

int museattn_gather_probe(const int32_t *table, const int32_t *seq_lens, const void *k_cache,
                          const void *v_cache, int page_size, int B, int table_stride,
                          int max_seq_len, int64_t num_rows, void *out, int work_groups,
                          void *stream) {
  if (!table || !seq_lens || !k_cache || !v_cache || !out) return MUSEATTN_ERR_NULL;
  if (page_size != 1 && page_size != 64) return MUSEATTN_ERR_PAGE_SIZE;
  if (B < 1 || B > MAX_BATCH || max_seq_len < 1 || max_seq_len > MAX_SEQ) return MUSEATTN_ERR_SHAPE;
  if ((int64_t)B * ((max_seq_len + CHUNK - 1) / CHUNK) >= (int64_t(1) << 31)) return MUSEATTN_ERR_SHAPE;
  if (num_rows < page_size || num_rows % page_size != 0 || num_rows >= (int64_t(1) << 32))
    return MUSEATTN_ERR_SHAPE;
  if ((int64_t)table_stride * page_size < max_seq_len || table_stride < 1) return MUSEATTN_ERR_TABLE;
  if (work_groups < 1 || work_groups > MAX_WORK_GROUPS) return MUSEATTN_ERR_PARAM;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(table, 4) ||
      !aligned(seq_lens, 4) || !aligned(out, 4))
    return MUSEATTN_ERR_ALIGN;
  (void)hipGetLastError();
  launch_gather_probe(table, seq_lens, static_cast<const uint8_t *>(k_cache),
                      static_cast<const uint8_t *>(v_cache), B, table_stride, max_seq_len,
                      page_size, num_rows, static_cast<uint32_t *>(out), work_groups,
                      static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? MUSEATTN_OK : MUSEATTN_ERR_LAUNCH;
}

namespace {
// The projection's own arguments (the gated output a is bf16 [T][1024]).
int check_oproj(const void *a, const void *o_weight, int T, int hidden, const void *y) {
  if (!a || !o_weight || !y) return MUSEATTN_ERR_NULL;
  if (T < 1 || hidden < 64 || hidden > MUSEATTN_MAX_HIDDEN || hidden % 64) return MUSEATTN_ERR_PARAM;
  if (!museattn::aligned(a, 16) || !museattn::aligned(o_weight, 16) || !museattn::aligned(y, 8))
    return MUSEATTN_ERR_ALIGN;
  const uintptr_t y0 = (uintptr_t)y, y1 = y0 + (uintptr_t)T * hidden * 2;
  const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)T * MUSEATTN_OUT_WIDTH * 2;
  const uintptr_t w0 = (uintptr_t)o_weight, w1 = w0 + (uintptr_t)hidden * MUSEATTN_OUT_WIDTH * 2;
  if ((y0 < a1 && a0 < y1) || (y0 < w1 && w0 < y1)) return MUSEATTN_ERR_ALIAS;
  return MUSEATTN_OK;
}
}  // namespace

int museattn_oproj(const void *a, const void *o_weight, int T, int hidden, void *y, void *stream) {
  const int st = check_oproj(a, o_weight, T, hidden, y);
  if (st != MUSEATTN_OK) return st;
  (void)hipGetLastError();
  museattn::launch_oproj(static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(o_weight),
                         static_cast<uint16_t *>(y), T, hidden, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? MUSEATTN_OK : MUSEATTN_ERR_LAUNCH;
}

int museattn_attn_step_oproj(const void *qkv, const int32_t *positions, const int32_t *table,
                             const int32_t *seq_lens, void *k_cache, void *v_cache, float kv_scale,
                             int page_size, int layer_kind, void *out, void *stream, int B, int L,
                             int table_stride, int max_seq_len, int64_t num_rows,
                             const museattn_params *params, void *workspace,
                             size_t workspace_bytes, const void *o_weight, int hidden, void *y,
                             void *oproj_start_event, void *oproj_end_event) {
  int st = museattn_check_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale,
                               page_size, layer_kind, out, B, L, table_stride, max_seq_len,
                               num_rows, params, workspace, workspace_bytes);
  if (st != MUSEATTN_OK) return st;
  const int T = B * L;
  st = check_oproj(out, o_weight, T, hidden, y);
  if (st != MUSEATTN_OK) return st;
  // y is written after the step: it must not overlap what the step reads or
  // writes either
  const uintptr_t y0 = (uintptr_t)y, y1 = y0 + (uintptr_t)T * hidden * 2;
  auto meets_y = [&](const void *p, uint64_t bytes) {
    const uintptr_t p0 = (uintptr_t)p, p1 = p0 + (uintptr_t)bytes;
    return y0 < p1 && p0 < y1;
  };
  if (meets_y(qkv, (uint64_t)T * MUSEATTN_QKV_WIDTH * 2) ||
      meets_y(k_cache, (uint64_t)num_rows * MUSEATTN_ROW_BYTES) ||
      meets_y(v_cache, (uint64_t)num_rows * MUSEATTN_ROW_BYTES) ||
      meets_y(workspace, workspace_bytes))
    return MUSEATTN_ERR_ALIAS;
  st = museattn_attn_step(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
                          layer_kind, out, stream, B, L, table_stride, max_seq_len, num_rows,
                          params, workspace, workspace_bytes);
  if (st != MUSEATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (oproj_start_event) (void)hipEventRecord(static_cast<hipEvent_t>(oproj_start_event), s);
  museattn::launch_oproj(static_cast<const uint16_t *>(out), static_cast<const uint16_t *>(o_weight),
                         static_cast<uint16_t *>(y), T, hidden, s);
  if (oproj_end_event) (void)hipEventRecord(static_cast<hipEvent_t>(oproj_end_event), s);
  return hipGetLastError() == hipSuccess ? MUSEATTN_OK : MUSEATTN_ERR_LAUNCH;
}

}  // extern "C"
