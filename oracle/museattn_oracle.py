"""CPU oracle for one gated grouped-query attention step over a paged FP8 E4M3 KV cache.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  The product path (the HIP library and
its Python binding in paged_fp8_kv_amd/) never imports, links or calls it, and
this module imports nothing from the product path.

What it computes is the operation of the task page "Gated attention decode
(muse_attention_decode)", section "What to compute", written out as a plain,
slow, float64 program (numpy matmul and exp are the only library steps).  For
each request b and block token j, at position p = positions[b*L + j]:
  1. the fused projection row is cut into query, key, value and gate heads;
  2. query and key heads are RMS-normalised with their weights, and the
     queries are multiplied by the q scale (5.473 on the page);
  3. on sliding-window layers both are rotated by position p;
  4. all the block's new key and value heads are rounded to fp8 and stored in
     their cache rows before any attention reads the cache;
  5. each query head takes a softmax of its scores (dot products with the
     cached keys of its KV head, divided by 8) over positions 0..p on a full
     layer or the last 2048 positions p-2047..p on a sliding one, and sums
     the matching cached values with those weights;
  6. each head's result is RMS-normalised with its weight, multiplied by the
     sigmoid of its gate, and returned as out [B, L, 16*64].
It also holds the output projection that follows the step in the decoder
layer (task page "Whole decoder layer", section "What to compute"; the
all-reduce after it is the identity on one GPU): y = out @ o^T, o [hidden,
1024].

Readings where the page is silent:
  * qkv row layout [q 16x64 | k 2x64 | v 2x64 | gate 16x64], head-major.
  * query head h reads KV head h // 8 (contiguous GQA groups of 8).
  * every rmsnorm carries a per-dimension weight of 64 values, used as given
    (x / sqrt(mean(x^2) + eps) * w); the output norm is per head over 64 dims.
  * RoPE is the half-split ("neox") rotation over all 64 dims, base 10000:
    pair (i, i+32) turns by theta_i = fp32(fp32(p) * fp32(base^(-i/32))).
  * FP8 is OCP E4M3FN (bias 7, no infinities, NaN = S.1111.111, max 448),
    round-to-nearest-even, saturating to +-448; one scalar kv_scale for K and
    V: stored byte = fp8(x / kv_scale), value read = decode(byte) * kv_scale.
    The rounding decision is taken on the fp32 value of x / kv_scale.
  * a verify block's token j sees the cached keys plus block tokens j' <= j,
    all read back from the cache as fp8.
  * the sliding window holds 2048 positions including the query's own.
  * paged addressing: row(b, u) = table[b][u // ps] * ps + u % ps; with page
    size 1 the table holds one cache row per position ("cache_loc").
"""
from __future__ import annotations

import math

import numpy as np

HQ = 16          # query heads per GPU shard (TP8)
HKV = 2          # key/value heads per GPU shard
D = 64           # head dim
GROUP = HQ // HKV
QKV_WIDTH = HQ * D + 2 * HKV * D + HQ * D   # 2304
Q_OFF, K_OFF, V_OFF, G_OFF = 0, HQ * D, HQ * D + HKV * D, HQ * D + 2 * HKV * D
FULL, SLIDING = 0, 1
WINDOW = 2048
SOFTMAX_DIV = 8.0   # the page divides q.K^T by 8 (= sqrt(64))


# --------------------------------------------------------------------------
# FP8 E4M3FN codec, written from the format definition (OCP 8-bit floating
# point specification, E4M3 encoding): 1 sign bit, 4 exponent bits (bias 7),
# 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111 is
# NaN; there is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448.
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3FN byte (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


# The 127 non-negative finite magnitudes in code order; the code order is the
# magnitude order, so a code's neighbours are the adjacent codes.
_POS_VALUES = e4m3_decode(np.arange(127))


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3FN byte, ties to the even code, saturating to +-448.

    The sign of x is kept, also when x rounds to zero (-tiny -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("e4m3_encode: NaN input")
    ax = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_POS_VALUES, ax, side="left")      # first value >= ax
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = ax - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(ax == _POS_VALUES[hi], hi, code)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


# value of every byte, for table-lookup dequantisation of long key ranges
_DECODE_TABLE = e4m3_decode(np.arange(256))


def e4m3_ordinal(codes) -> np.ndarray:
    """Signed position of a code on the E4M3 number line (+0 and -0 both 0).

    Two codes are within k ulp of each other iff their ordinals differ by <= k."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


# --------------------------------------------------------------------------
# Elementwise pieces of the step ("What to compute" listing).
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis (64 dims)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(w, dtype=np.float64)


def rope_inv_freq(base: float) -> np.ndarray:
    """fp32 inverse frequencies base^(-i/32), i = 0..31, as float64 values."""
    i = np.arange(D // 2, dtype=np.float64)
    return (float(base) ** (-i / (D // 2))).astype(np.float32).astype(np.float64)


def rope_angles(p: int, base: float) -> np.ndarray:
    """theta_i = fp32(fp32(p) * inv_i), returned as float64 (exact fp32 values)."""
    inv = rope_inv_freq(base).astype(np.float32)
    return (np.float32(p) * inv).astype(np.float32).astype(np.float64)


def rope_neox(x: np.ndarray, p: int, base: float) -> np.ndarray:
    """Half-split rotation: (x_i, x_{i+32}) -> (x_i c - x_{i+32} s, x_{i+32} c + x_i s)."""
    x = np.asarray(x, dtype=np.float64)
    th = rope_angles(p, base)
    c, s = np.cos(th), np.sin(th)
    a, b = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def cache_row(table: np.ndarray, b: int, u, page_size: int):
    """Cache row of request b's position u: table[b][u // ps] * ps + u % ps."""
    u = np.asarray(u, dtype=np.int64)
    return table[b, u // page_size].astype(np.int64) * page_size + u % page_size


# --------------------------------------------------------------------------
# The step, in the listing's order.
# --------------------------------------------------------------------------

def prologue(qkv, positions, w_q, w_k, *, eps, q_scale, rope: bool, rope_base, kv_scale):
    """Split, QK-norm, RoPE and fp8 quantisation of the new k and v.

    qkv: float values of the bf16 rows [T, 2304].  Returns
      q     float64 [T, 16, 64]  (rmsnorm(q) * w_q * q_scale, rotated if rope)
      kbyte uint8   [T, 2, 64]   fp8(k / kv_scale)
      vbyte uint8   [T, 2, 64]   fp8(v / kv_scale)
      gate  float64 [T, 16, 64]
    """
    x = np.asarray(qkv, dtype=np.float64)
    T = x.shape[0]
    q = x[:, Q_OFF:Q_OFF + HQ * D].reshape(T, HQ, D)
    k = x[:, K_OFF:K_OFF + HKV * D].reshape(T, HKV, D)
    v = x[:, V_OFF:V_OFF + HKV * D].reshape(T, HKV, D)
    gate = x[:, G_OFF:G_OFF + HQ * D].reshape(T, HQ, D)
    q = rmsnorm(q, w_q, eps) * float(q_scale)
    k = rmsnorm(k, w_k, eps)
    if rope:
        q = np.stack([rope_neox(q[t], int(positions[t]), rope_base) for t in range(T)])
        k = np.stack([rope_neox(k[t], int(positions[t]), rope_base) for t in range(T)])
    ks = float(kv_scale)
    kbyte = e4m3_encode((k / ks).astype(np.float32))
    vbyte = e4m3_encode((v / ks).astype(np.float32))
    return q, kbyte, vbyte, gate


def write_rows(k_pool, v_pool, table, positions, B, L, page_size, kbyte, vbyte):
    """cache[row(b, p_t)] = fp8(k_t), fp8(v_t) for every block token t."""
    for b in range(B):
        for j in range(L):
            t = b * L + j
            r = int(cache_row(table, b, int(positions[t]), page_size))
            k_pool[r] = kbyte[t]
            v_pool[r] = vbyte[t]


def visible_keys(p: int, window: int | None) -> tuple[int, int]:
    """Inclusive key-position range a query at position p attends to."""
    lo = 0 if window is None else max(0, p - (window - 1))
    return lo, p


def attend(q, k_pool, v_pool, table, positions, B, L, page_size, kv_scale, window, tokens=None):
    """a = softmax(q . K^T / 8) . V per (token, head), two passes, float64.

    K and V are read through the table from the pools (anything indexable by an
    int64 row array giving [n, 2, 64] bytes) and dequantised as decode*kv_scale.
    window=None attends to every key 0..p, else to the last `window` positions.
    tokens: block-token indices j to compute (None = all); the others stay 0.
    Returns a float64 [B*L, 16, 64]."""
    q = np.asarray(q, dtype=np.float64)
    ks = float(kv_scale)
    a = np.zeros((B * L, HQ, D))
    for b in range(B):
        # the union of the block tokens' key ranges, read and dequantised once
        spans = [visible_keys(int(positions[b * L + j]), window) for j in range(L)]
        ulo = min(lo for lo, _ in spans)
        uhi = max(hi for _, hi in spans)
        rows = cache_row(table, b, np.arange(ulo, uhi + 1), page_size)
        kd = _DECODE_TABLE[k_pool[rows]] * ks          # [n, 2, 64]
        vd = _DECODE_TABLE[v_pool[rows]] * ks
        for j in (range(L) if tokens is None else tokens):
            t = b * L + j
            lo, hi = spans[j]
            kj, vj = kd[lo - ulo:hi - ulo + 1], vd[lo - ulo:hi - ulo + 1]
            for h in range(HQ):
                g = h // GROUP
                s = kj[:, g, :] @ q[t, h] / SOFTMAX_DIV
                m = np.max(s)
                e = np.exp(s - m)
                a[t, h] = (e @ vj[:, g, :]) / np.sum(e)
    return a


def gated_output(a, gate, w_o, eps):
    """out = rmsnorm(a) * w_o * sigmoid(gate), per head; float64 [T, 16, 64]."""
    return rmsnorm(a, w_o, eps) * sigmoid(gate)


def attn_step(qkv, positions, table, k_pool, v_pool, *, B, L, page_size, layer_kind,
              kv_scale, w_q, w_k, w_o, eps, q_scale, rope_base=10000.0, window=WINDOW,
              new_rows=None, tokens=None):
    """The whole step.  Writes the new rows into k_pool / v_pool (in place).

    new_rows: optional (kbyte, vbyte) to write instead of the oracle's own
    quantised k, v -- used to attend to another implementation's written
    entries, as the page's correctness section does for the cache check.
    tokens: block-token indices whose outputs are computed (None = all; the
    others are left 0) -- the new rows of every token are written regardless.
    Returns (out float64 [B, L, 16*64], kbyte, vbyte)."""
    sliding = layer_kind == SLIDING
    q, kbyte, vbyte, gate = prologue(qkv, positions, w_q, w_k, eps=eps, q_scale=q_scale,
                                     rope=sliding, rope_base=rope_base, kv_scale=kv_scale)
    wk, wv = (kbyte, vbyte) if new_rows is None else new_rows
    write_rows(k_pool, v_pool, table, positions, B, L, page_size, wk, wv)
    a = attend(q, k_pool, v_pool, table, positions, B, L, page_size, kv_scale,
               window if sliding else None, tokens)
    out = gated_output(a, gate, w_o, eps)
    return out.reshape(B, L, HQ * D), kbyte, vbyte


def oproj(a, o_weight):
    """The attention output projection: y[t, n] = sum_k a[t, k] * o[n, k]
    (a [T, 1024], o [hidden, 1024]); float64."""
    a = np.asarray(a, dtype=np.float64)
    o_weight = np.asarray(o_weight, dtype=np.float64)
    return a @ o_weight.T
