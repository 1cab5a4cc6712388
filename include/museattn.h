/*
 * libmuseattn -- one attention step of gated grouped-query attention over a
 * paged FP8 E4M3 KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined on the task page "Gated attention decode
 * (muse_attention_decode)", section "What to compute" (the window and the
 * causal rule come from its section "Shapes"; blocks of more than 8 tokens
 * are the attention part of the prefill task page "Prefill layer", section
 * "Shapes", over the same cache).  One call serves B requests of L block
 * tokens each: a decode step (L = 1), a causal verify block (L <= 8) or a
 * causal prefill block (up to 16384 tokens).  For block token j of request b,
 * at position p = positions[b*L + j]:
 *   1. its bf16 row of the fused projection is cut into 16 query heads, 2 key
 *      heads, 2 value heads and 16 gate heads of 64 values each;
 *   2. every query and key head is RMS-normalised over its 64 values and
 *      multiplied by a per-dimension weight; the queries are then scaled by
 *      q_scale;
 *   3. on sliding-window layers the query and key heads are rotated by the
 *      angle set of position p (half-split rotary embedding);
 *   4. its key and value heads, divided by kv_scale and rounded to E4M3, are
 *      stored in the token's cache row;
 *   5. query head h attends to KV head h / 8 with scores scaled by 1/8, over
 *      the cached keys at positions 0..p on a full layer or p-2047..p on a
 *      sliding one (the block's own new rows included, read back from the
 *      cache);
 *   6. each head's attention result is RMS-normalised, multiplied by its
 *      weight and by the logistic sigmoid of the head's gate, and stored as
 *      bf16.
 *
 * Shapes per GPU shard (section "Shapes"): 16 query heads, 2 KV heads, head
 * dim 64; query head h reads KV head h / 8.  The fused row is bf16
 * [q 16x64 | k 2x64 | v 2x64 | gate 16x64] = 2304 values.
 *
 * Paged cache (section "Shapes": E4M3 bytes, page size 1 or 64, a scale of
 * 1 or 1/64): k_cache and v_cache are separate byte arrays of num_rows rows;
 * a row holds one token's two KV heads, [2][64] E4M3FN bytes = 128 B.  With
 * page size ps, row(b, u) = table[b*table_stride + u/ps]*ps + u%ps: at ps = 1
 * the table holds one cache row per position ("cache_loc"); at ps = 64 it
 * holds page ids and a page is 64 consecutive rows.  The new tokens' rows are
 * found through the same table, so the caller allocates them (as a serving
 * engine does) before the call.
 *
 * Call contract (section "Rules": CUDA graphs, fresh inputs):
 *  - every pointer argument except `params` and `stream` is DEVICE memory
 *    owned by the caller; `params` is a host struct read during the call.
 *  - the library never allocates, frees, synchronises or reads device values
 *    on the host; all work is enqueued on `stream`, so a call can be captured
 *    into a HIP graph.  Nothing is cached between calls.
 *  - k_cache / v_cache are written only at the B*L new rows.  The buffers
 *    the step writes (out, k_cache and v_cache of num_rows rows each, the
 *    workspace) must not overlap one another or any buffer it reads (qkv,
 *    positions, table, seq_lens, the norm weights); `workspace` holds scratch
 *    data of one call (it must not be shared by calls that may run
 *    concurrently).
 *  - device-side indices are clamped into the extents the host validated
 *    (rows into [0, num_rows), positions into [0, max_seq_len)), so
 *    inconsistent device data gives wrong numbers, never an out-of-bounds
 *    access.  seq_lens[b] must not exceed max_seq_len; keys beyond it are not
 *    attended.
 *
 * Errors: 0 on success; a negative museattn_status if host-side validation
 * fails, in which case nothing was enqueued; MUSEATTN_ERR_LAUNCH if a kernel
 * launch reported an error (hipGetLastError).
 */
#ifndef MUSEATTN_H
#define MUSEATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUSEATTN_ABI_VERSION 1

/* Layer kinds (task page, section "Shapes"): a full-attention layer sees the
 * whole context and uses no RoPE; a sliding-window layer sees the last 2048
 * positions (the query's own included) and rotates q and k. */
enum museattn_layer_kind { MUSEATTN_FULL = 0, MUSEATTN_SLIDING = 1 };

#define MUSEATTN_WINDOW 2048
#define MUSEATTN_QKV_WIDTH 2304
#define MUSEATTN_OUT_WIDTH 1024
#define MUSEATTN_ROW_BYTES 128
#define MUSEATTN_MAX_HIDDEN 65536   /* o-projection output features */

enum museattn_status {
  MUSEATTN_OK = 0,
  MUSEATTN_ERR_NULL = -1,         /* a required pointer is null */
  MUSEATTN_ERR_PAGE_SIZE = -2,    /* page_size is not 1 or 64 */
  MUSEATTN_ERR_LAYER_KIND = -3,   /* layer_kind is not FULL or SLIDING */
  MUSEATTN_ERR_SHAPE = -4,        /* B (1..1024), L (1..16384), B * ceil(L / 16)
                                     (L > 8) above 4096, max_seq_len, num_rows
                                     (a multiple of page_size below 2^32) out
                                     of range, or a plan whose chunk count
                                     could reach 2^31 (B * ceil(max_seq_len /
                                     32) roughly, per 16-token group beyond
                                     L = 8) */
  MUSEATTN_ERR_TABLE = -5,        /* table_stride < ceil(max_seq_len / page_size) */
  MUSEATTN_ERR_ALIGN = -6,        /* k_cache, v_cache, qkv or a norm weight not
                                     16-byte aligned, out not 8-byte aligned,
                                     positions/table/seq_lens not 4-byte aligned */
  MUSEATTN_ERR_WORKSPACE = -7,    /* workspace smaller than museattn_workspace_bytes()
                                     or not 256-byte aligned */
  MUSEATTN_ERR_PARAM = -8,        /* kv_scale, eps, q_scale, rope_base or
                                     work_groups out of range */
  MUSEATTN_ERR_ALIAS = -9,        /* a buffer the step writes (out, k_cache,
                                     v_cache, workspace) overlaps another one
                                     of them or one it reads (qkv, positions,
                                     table, seq_lens, a norm weight) */
  MUSEATTN_ERR_LAUNCH = -10       /* a kernel launch failed */
};

/* Constants of the step that the page fixes or that the computation needs
 * but the page's input list leaves implicit (all read on the host). */
typedef struct museattn_params {
  const float *q_norm_w;   /* device float32 [64], 16-byte aligned: per-dim weight of
                              q's rmsnorm */
  const float *k_norm_w;   /* device float32 [64], 16-byte aligned: per-dim weight of
                              k's rmsnorm */
  const float *o_norm_w;   /* device float32 [64], 16-byte aligned: per-dim weight of
                              the output rmsnorm */
  float eps;               /* rmsnorm epsilon, >= 0 (1e-6) */
  float q_scale;           /* multiplier of the normed q (5.473) */
  float rope_base;         /* RoPE base, > 0 (10000) */
  int work_groups;         /* attention work-groups, each taking an equal share
                              of all requests' key chunks; 0 = chosen from the
                              shapes, else 1..65535.  Changes only the
                              summation order. */
} museattn_params;

/* Bytes of device workspace museattn_attn_step needs for these shapes (a
 * function of its arguments only).  Returns 0 if the arguments are invalid. */
size_t museattn_workspace_bytes(int B, int L, int max_seq_len, int page_size, int layer_kind,
                                const museattn_params *params);

/* Host-side validation of museattn_attn_step's arguments, without touching
 * the device (pointers are checked for null, alignment and overlap only).
 * Returns MUSEATTN_OK or the status museattn_attn_step would return. */
int museattn_check_args(const void *qkv, const int32_t *positions, const int32_t *table,
                        const int32_t *seq_lens, const void *k_cache, const void *v_cache,
                        float kv_scale, int page_size, int layer_kind, const void *out,
                        int B, int L, int table_stride, int max_seq_len, int64_t num_rows,
                        const museattn_params *params, const void *workspace,
                        size_t workspace_bytes);

/* One attention step (the operation described at the top of this file).
 *   qkv        bf16 [B*L][2304], row t = b*L + j, 16-byte aligned
 *   positions  int32 [B*L], p of token t (normally seq_lens[b] - L + j)
 *   table      int32 [B][table_stride]: rows (page_size 1) or page ids (64)
 *   seq_lens   int32 [B]: cached tokens + L ("FA3 lengths"), <= max_seq_len
 *   k_cache,
 *   v_cache    E4M3FN bytes [num_rows][2][64], 16-byte aligned; the B*L
 *              rows row(b, positions[t]) are written, all other rows read-only
 *   kv_scale   > 0: stored byte = fp8(x / kv_scale); read value = byte * kv_scale
 *   page_size  1 or 64
 *   layer_kind MUSEATTN_FULL or MUSEATTN_SLIDING
 *   out        bf16 [B][L][1024], 8-byte aligned
 *   stream     hipStream_t the work is enqueued on (NULL = default stream)
 *   1 <= B <= 1024, 1 <= L <= 16384 with B * ceil(L / 16) <= 4096 when L > 8
 *   (up to 8 block tokens the new rows are written inside the attention
 *   kernel; beyond, a first kernel writes them all),
 *   table_stride >= ceil(max_seq_len / page_size),
 *   L <= max_seq_len <= 2^30, num_rows a multiple of page_size,
 *   workspace  device scratch of >= museattn_workspace_bytes(...) bytes,
 *              256-byte aligned. */
int museattn_attn_step(const void *qkv, const int32_t *positions, const int32_t *table,
                       const int32_t *seq_lens, void *k_cache, void *v_cache, float kv_scale,
                       int page_size, int layer_kind, void *out, void *stream, int B, int L,
                       int table_stride, int max_seq_len, int64_t num_rows,
                       const museattn_params *params, void *workspace, size_t workspace_bytes);

/* museattn_attn_step that also records two caller-created hipEvent_t on
 * `stream`, immediately before and after the split-K attention kernel (the
 * step's dominant kernel), so a profiler of the caller can time that kernel
 * alone.  Either event may be NULL (not recorded).  Same arguments, effects
 * and statuses as museattn_attn_step. */
int museattn_attn_step_profiled(const void *qkv, const int32_t *positions, const int32_t *table,
                                const int32_t *seq_lens, void *k_cache, void *v_cache,
                                float kv_scale, int page_size, int layer_kind, void *out,
                                void *stream, int B, int L, int table_stride, int max_seq_len,
                                int64_t num_rows, const museattn_params *params, void *workspace,
                                size_t workspace_bytes, void *attn_start_event,
                                void *attn_end_event);

/* Bytes of the library's static device scratch (museattn_attn_step_noalloc). */
#define MUSEATTN_STATIC_SCRATCH_BYTES (32u << 20)

/* museattn_attn_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments as museattn_attn_step without the workspace:
 * the step's scratch (plan and split-K partials) lives in a fixed device array
 * of MUSEATTN_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends.  The call allocates and frees nothing; its first call on a
 * device looks up that array's address there (hipGetSymbolAddress, with the
 * stream's device current) and keeps it.
 *   - Shapes whose museattn_workspace_bytes(...) exceeds the array are
 *     rejected with MUSEATTN_ERR_WORKSPACE (32 MiB holds every decode shape,
 *     verify blocks of L = 8 up to B = 736, prefill blocks up to about 240
 *     16-token groups).
 *   - Every call on one GPU shares the array: calls that may overlap in time
 *     on one GPU (other streams, concurrent graph replays) race and must be
 *     serialised by the caller.  Each call rewrites all it reads of the array,
 *     so nothing needs clearing between calls.
 * Statuses: those of museattn_attn_step (MUSEATTN_ERR_LAUNCH also if the
 * array's address cannot be looked up). */
int museattn_attn_step_noalloc(const void *qkv, const int32_t *positions, const int32_t *table,
                               const int32_t *seq_lens, void *k_cache, void *v_cache,
                               float kv_scale, int page_size, int layer_kind, void *out,
                               void *stream, int B, int L, int table_stride, int max_seq_len,
                               int64_t num_rows, const museattn_params *params);

/* The attention output projection of the decoder layer (task page "Whole
 * decoder layer", section "What to compute": the gated attention output times
 * o^T; on one GPU the all-reduce that follows is the identity):
 *   y[t][n] = sum_k a[t][k] * o_weight[n][k],   k < 1024 (16 heads x 64 dims),
 * bf16 operands, fp32 accumulation, bf16 y (round to nearest even).
 *   a         bf16 [T][1024], 16-byte aligned (the step's `out`)
 *   o_weight  bf16 [hidden][1024], row n = output feature n, 16-byte aligned
 *   T         >= 1 tokens
 *   hidden    output features, a multiple of 64 in [64, MUSEATTN_MAX_HIDDEN]
 *   y         bf16 [T][hidden], 8-byte aligned, overlapping neither a nor o_weight
 *   stream    hipStream_t the work is enqueued on
 * Device pointers, owned by the caller.  Up to 63 tokens a kernel that keeps
 * rows of o in registers runs; from 64 tokens on, an LDS-tiled MFMA GEMM
 * whose tile shape is chosen from T and hidden.
 * Either way the call allocates nothing and keeps nothing between calls, so
 * any call (a shape's first included) can be captured into a graph.
 * Statuses: MUSEATTN_ERR_NULL, _PARAM (T or hidden), _ALIGN, _ALIAS, _LAUNCH. */
int museattn_oproj(const void *a, const void *o_weight, int T, int hidden, void *y, void *stream);

/* museattn_attn_step followed by museattn_oproj on its output, on the same
 * stream (the step's `out` still receives the gated output; the projection
 * reads it back from the cache hierarchy).  The two optional caller-created
 * hipEvent_t are recorded around the projection kernel.  Checks both calls'
 * arguments before enqueuing anything (y must also not overlap qkv, the
 * caches or the workspace). */
int museattn_attn_step_oproj(const void *qkv, const int32_t *positions, const int32_t *table,
                             const int32_t *seq_lens, void *k_cache, void *v_cache, float kv_scale,
                             int page_size, int layer_kind, void *out, void *stream, int B, int L,
                             int table_stride, int max_seq_len, int64_t num_rows,
                             const museattn_params *params, void *workspace,
                             size_t workspace_bytes, const void *o_weight, int hidden, void *y,
                             void *oproj_start_event, void *oproj_end_event);

/* A memory-system probe, not part of the step: reads the K and V rows of
 * every key position 0 .. seq_lens[b] - 1 of every request (the keys a
 * full-layer decode step attends to) through the table, each key once, with
 * nothing else to do: work_groups work-groups of 8 waves take equal shares of
 * all requests' keys laid end to end, stage their row ids in LDS and stream
 * the rows with 128-byte-row loads.  It writes one XOR checksum of the rows'
 * 32-bit words per work-group to out (uint32 [work_groups], device).  Its
 * duration is the time this part needs to gather the step's rows: the
 * ceiling of the attention kernel on this workload.  Arguments as in
 * museattn_attn_step; 1 <= work_groups <= 65535.  Statuses:
 * MUSEATTN_ERR_NULL, _PAGE_SIZE, _SHAPE, _TABLE, _PARAM, _ALIGN, _LAUNCH. */
int museattn_gather_probe(const int32_t *table, const int32_t *seq_lens, const void *k_cache,
                          const void *v_cache, int page_size, int B, int table_stride,
                          int max_seq_len, int64_t num_rows, void *out, int work_groups,
                          void *stream);

/* Attention work-groups the library launches for these shapes
 * (params->work_groups = 0 chooses). */
int museattn_work_groups(int B, int L, int max_seq_len, int layer_kind, const museattn_params *params);

/* Static description of a status code. */
const char *museattn_strerror(int status);

/* MUSEATTN_ABI_VERSION of the built library. */
int museattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUSEATTN_H */
