"""Seeded synthetic workloads for the attention step (inputs only).

This module draws the inputs that both the HIP path and the CPU oracle consume:
the fused projection rows, norm weights, positions, FA3-style sequence lengths,
the cache-row / page table and the bytes already in the paged FP8 cache.  It
holds none of the step's arithmetic: no norm, rotation, attention or fp8
rounding of new entries.  The bytes of the cached (old) tokens are produced by
PyTorch's own float8_e4m3fn cast of clipped N(0,1) draws, a library routine.

Shapes follow the task page "Gated attention decode (muse_attention_decode)",
section "Shapes": 16 query heads and 2 KV heads of dim 64 per GPU, decode
(L = 1) or an 8-token verify block, contexts around 80K, page size 1 or 64,
kv_scale 1 or 1/64.  The page's "spread" and "dist" input families are not
defined beyond a sentence each; the draws below stand in for them:
  soft       cached K and V elements are clipped N(0,1) draws;
  coherent   (section "Correctness": each head's keys share a direction, so
             attention spreads over many keys; on full layers the values of the
             low-attention keys share a direction too) -- per request and KV
             head, keys are 8 d + 0.1 z and, on full layers, values are
             8 w + 0.5 z, for unit vectors d, w and z ~ N(0,1) per element;
  edges      (section "Correctness": keys at the window's edges) -- soft draws,
             with the keys and values at the edges of the visible range
             enlarged 6-fold (clipped): on sliding layers the first visible
             position of each block token's window and the one just outside
             it, on full layers positions 0 and 1; on both, the last two cached
             positions;
  outliers   (named by the prefill page's tests, not defined there) -- soft
             draws with one key element in 64 enlarged 8-fold (then clipped):
             extreme scores for the softmax; values stay soft (an outlier
             value can put a head's output near 8 after the output norm,
             where bf16 rounding alone exceeds the output bar).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

HQ, HKV, D = 16, 2, 64
QKV_WIDTH = 2304
ROW_BYTES = HKV * D        # bytes of one cache row per tensor (both KV heads)
FULL, SLIDING = 0, 1
SENTINEL = 0x7F            # E4M3 NaN: marks rows nobody may read before writing
_CLIP = 6.9                # |x| <= 6.9 keeps 64*x below the format's 448


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    L: int
    layer_kind: int
    page_size: int
    kv_scale: float          # exactly representable in fp32
    ctx: np.ndarray          # int64 [B] cached tokens per request
    num_rows: int            # rows in each of the K and V pools
    qkv: torch.Tensor        # bf16 [B*L, 2304] (CPU)
    w_q: np.ndarray          # float32 [64]
    w_k: np.ndarray
    w_o: np.ndarray
    table: np.ndarray        # int32 [B, table_stride]; unused slots = -1
    pages: list = field(default_factory=list)  # per request: int64 page (or row) ids in order
    origin: list = field(default_factory=list)  # request ids in the workload drawn (subsets)
    dist: str = "soft"       # "soft", "coherent" or "edges" (module docstring)

    @property
    def T(self) -> int:
        return self.B * self.L

    @property
    def seq_lens(self) -> np.ndarray:
        return (self.ctx + self.L).astype(np.int32)

    @property
    def positions(self) -> np.ndarray:
        return (self.ctx[:, None] + np.arange(self.L)[None, :]).reshape(-1).astype(np.int32)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    @property
    def table_stride(self) -> int:
        return int(self.table.shape[1])

    @property
    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes the step reads: 256 B per visible key position."""
        span = self.seq_lens.astype(np.int64)
        if self.layer_kind == SLIDING:
            first = self.ctx.astype(np.int64)  # position of block token 0
            lo = np.maximum(0, first - 2047)
            span = self.seq_lens.astype(np.int64) - lo
        return int(span.sum()) * 2 * ROW_BYTES

    @property
    def attn_flops(self) -> int:
        """Algorithmic FLOPs of the attention: 4 * 64 per (visible key, token, head)
        (q.k and p.v, a multiply and an add each)."""
        p = self.positions.astype(np.int64)
        keys = p + 1 if self.layer_kind == FULL else np.minimum(p + 1, 2048)
        return int(keys.sum()) * HQ * D * 4

    def subset(self, requests) -> "Workload":
        """The same draws restricted to some requests (their pool placement kept)."""
        req = [int(b) for b in requests]
        sub = Workload(name=f"{self.name}[{len(req)} of {self.B}]", seed=self.seed, B=len(req),
                       L=self.L, layer_kind=self.layer_kind, page_size=self.page_size,
                       kv_scale=self.kv_scale, ctx=self.ctx[req].copy(), num_rows=self.num_rows,
                       qkv=self.qkv.view(self.B, self.L, QKV_WIDTH)[req].reshape(-1, QKV_WIDTH).clone(),
                       w_q=self.w_q, w_k=self.w_k, w_o=self.w_o, table=self.table[req].copy(),
                       pages=[self.pages[b] for b in req],
                       origin=[self.origin[b] if self.origin else b for b in req], dist=self.dist)
        return sub

    def cache_values(self, b: int) -> tuple[np.ndarray, np.ndarray]:
        """Bytes of request b's cached positions 0..ctx_b-1: K, V uint8 [ctx_b, 2, 64]."""
        n = int(self.ctx[b])
        src = self.origin[b] if self.origin else b
        rng = np.random.Generator(np.random.PCG64([self.seed, src]))
        x = rng.standard_normal(2 * n * ROW_BYTES, dtype=np.float32)
        if self.dist == "coherent":
            x = x.reshape(2, n, HKV, D)
            rd = np.random.Generator(np.random.PCG64([self.seed, src, 1]))
            dirs = rd.standard_normal((2, HKV, D))
            dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
            x[0] = 8.0 * dirs[0][None] + 0.1 * x[0]
            if self.layer_kind == FULL:
                x[1] = 8.0 * dirs[1][None] + 0.5 * x[1]
            x = x.reshape(-1).astype(np.float32)
        elif self.dist == "edges":
            x = x.reshape(2, n, HKV, D)
            first = int(self.ctx[b])          # position of block token 0
            if self.layer_kind == SLIDING:
                edge = [first - 2048 + j for j in range(self.L + 1)]
            else:
                edge = [0, 1]
            edge += [n - 2, n - 1]
            for u in sorted({u for u in edge if 0 <= u < n}):
                x[:, u] *= 6.0
            x = x.reshape(-1)
        elif self.dist == "outliers":
            ro = np.random.Generator(np.random.PCG64([self.seed, src, 2]))
            x = x.reshape(2, -1)
            pick = ro.random(x.shape[1]) < 1.0 / 64.0
            x[0] = np.where(pick, x[0] * 8.0, x[0])
            x = x.reshape(-1)
        elif self.dist != "soft":
            raise ValueError(f"unknown distribution {self.dist!r}")
        np.clip(x, -_CLIP, _CLIP, out=x)
        xt = torch.from_numpy(x)
        if self.kv_scale != 1.0:
            xt = xt / self.kv_scale     # power-of-two scales: exact
        byt = xt.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(2, n, HKV, D)
        return byt[0], byt[1]


def _stream(seed: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, (1 << 20) + tag]))


def make(name: str, seed: int, B: int, L: int, ctx, layer_kind: int, page_size: int,
         kv_scale: float, pool_rows: int | None = None, dist: str = "soft") -> Workload:
    """Draw one workload.  ctx: int, or (lo, hi) for a uniform draw per request;
    dist: the cached K/V distribution (module docstring)."""
    if isinstance(ctx, tuple):
        ctx_arr = _stream(seed, 3).integers(ctx[0], ctx[1] + 1, size=B).astype(np.int64)
    else:
        ctx_arr = np.full(B, int(ctx), dtype=np.int64)
    seq = ctx_arr + L
    T = B * L
    rq = _stream(seed, 0)
    qkv = torch.from_numpy(rq.standard_normal((T, QKV_WIDTH), dtype=np.float32)).to(torch.bfloat16)
    rw = _stream(seed, 1)
    w = (1.0 + 0.1 * rw.standard_normal((3, D))).astype(np.float32)

    ps = page_size
    units_per_req = [int((s + ps - 1) // ps) for s in seq]        # pages (or rows) per request
    need = sum(units_per_req)
    if pool_rows is None:
        pool_units = 2 * need + 1
    else:
        pool_units = pool_rows // ps
    if pool_units < need + 1:
        raise ValueError(f"pool of {pool_units} units cannot hold {need} + 1 poison unit")
    rt = _stream(seed, 2)
    # distinct random units from [0, pool_units - 1); the last unit is a poison
    # unit (sentinel bytes) that unused table slots point at.
    chosen = rt.choice(pool_units - 1, size=need, replace=False).astype(np.int64)
    stride = max(units_per_req)
    table = np.full((B, stride), -1, dtype=np.int32)
    pages = []
    off = 0
    for b in range(B):
        n = units_per_req[b]
        table[b, :n] = chosen[off:off + n]
        pages.append(chosen[off:off + n])
        off += n
    return Workload(name=name, seed=seed, B=B, L=L, layer_kind=layer_kind, page_size=ps,
                    kv_scale=float(np.float32(kv_scale)), ctx=ctx_arr,
                    num_rows=pool_units * ps, qkv=qkv, w_q=w[0], w_k=w[1], w_o=w[2],
                    table=table, pages=pages, dist=dist)


# The five workloads of record (seed = 1000 + id); config 3 runs both layer kinds.
def config(cid: str, pool_rows: int | None = None) -> Workload:
    if cid == "0":
        return make("tiny-full-decode", 1000, 1, 1, 512, FULL, 1, 1.0, pool_rows or 4096)
    if cid == "1":
        return make("sliding-decode-ctx80k", 1001, 1, 1, 80000, SLIDING, 1, 1.0, pool_rows)
    if cid == "2":
        # ~80 GB of K+V rows in all (two pools of 312.5M rows of 128 B)
        return make("full-decode-b32-ctx60k-100k", 1002, 32, 1, (60000, 100000), FULL, 1, 1.0,
                    pool_rows or 312_500_000)
    if cid == "3s":
        return make("verify-L8-sliding-ctx80k", 1003, 1, 8, 80000, SLIDING, 1, 1.0, pool_rows)
    if cid == "3f":
        return make("verify-L8-full-ctx80k", 1003, 1, 8, 80000, FULL, 1, 1.0, pool_rows)
    if cid == "4":
        return make("paged64-full-decode-b16-kvscale1/64", 1004, 16, 1, (60000, 100000), FULL,
                    64, 1.0 / 64, pool_rows)
    # prefill blocks (the prefill task page's scored shapes; seed 1100 + index)
    prefill = {
        "pf1f": ("prefill-turn1-full-ctx80k-L753", 1, 80000, 753, FULL),
        "pf1s": ("prefill-turn1-sliding-ctx80k-L753", 1, 80000, 753, SLIDING),
        "pf4f": ("prefill-turn4-full-b4-ctx80k-L753", 4, 80000, 753, FULL),
        "pf4s": ("prefill-turn4-sliding-b4-ctx80k-L753", 4, 80000, 753, SLIDING),
        "pff0": ("prefill-first-full-ctx0-L16384", 1, 0, 16384, FULL),
        "pfs32": ("prefill-first-sliding-ctx32k-L16384", 1, 32768, 16384, SLIDING),
        "pff32": ("prefill-first-full-ctx32k-L16384", 1, 32768, 16384, FULL),
        "pff64": ("prefill-first-full-ctx64k-L16384", 1, 65536, 16384, FULL),
    }
    if cid in prefill:
        name, B, ctx, L, kind = prefill[cid]
        return make(name, 1100 + list(prefill).index(cid), B, L, ctx, kind, 1, 1.0, pool_rows)
    # the decode page's batch shapes (its floor table): contexts spread over
    # [60000, 100000], page size 1, pools just large enough (seed 1200 + index)
    batch = {
        "d16s": ("decode-b16-sliding-ctx60k-100k", 16, 1, SLIDING),
        "d16f": ("decode-b16-full-ctx60k-100k", 16, 1, FULL),
        "d32s": ("decode-b32-sliding-ctx60k-100k", 32, 1, SLIDING),
        "v16s": ("verify-b16-L8-sliding-ctx60k-100k", 16, 8, SLIDING),
        "v16f": ("verify-b16-L8-full-ctx60k-100k", 16, 8, FULL),
        "v32s": ("verify-b32-L8-sliding-ctx60k-100k", 32, 8, SLIDING),
        "v32f": ("verify-b32-L8-full-ctx60k-100k", 32, 8, FULL),
    }
    if cid in batch:
        name, B, L, kind = batch[cid]
        return make(name, 1200 + list(batch).index(cid), B, L, (60000, 100000), kind, 1, 1.0,
                    pool_rows)
    raise KeyError(cid)


CONFIG_IDS = ("0", "1", "2", "3s", "3f", "4")
PREFILL_IDS = ("pf1f", "pf1s", "pf4f", "pf4s", "pff0", "pfs32", "pff32", "pff64")
BATCH_IDS = ("d16s", "d16f", "d32s", "v16s", "v16f", "v32s", "v32f")


# --------------------------------------------------------------------------
# Pool construction (plumbing).  Rows of a request's unit i hold positions
# i*ps .. i*ps+ps-1; the generator places them unit by unit.
# --------------------------------------------------------------------------

def _unit_blocks(w: Workload, b: int, kb: np.ndarray):
    """Request b's cached bytes padded to whole units: [units, ps, 2, 64]."""
    ps = w.page_size
    n_units = len(w.pages[b])
    out = np.full((n_units * ps, HKV, D), SENTINEL, dtype=np.uint8)
    out[: kb.shape[0]] = kb
    return out.reshape(n_units, ps, HKV, D)


def build_pools_numpy(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Host pools [num_rows, 2, 64]: cached rows filled, every other row sentinel."""
    ps = w.page_size
    kp = np.full((w.num_rows // ps, ps, HKV, D), SENTINEL, dtype=np.uint8)
    vp = np.full_like(kp, SENTINEL)
    for b in range(w.B):
        kb, vb = w.cache_values(b)
        kp[w.pages[b]] = _unit_blocks(w, b, kb)
        vp[w.pages[b]] = _unit_blocks(w, b, vb)
    return kp.reshape(w.num_rows, HKV, D), vp.reshape(w.num_rows, HKV, D)


def build_pools_device(w: Workload, device, fill_all: bool | None = None):
    """Device pools (torch uint8 [num_rows, 2, 64]).

    Large pools are left uninitialised except for the rows the step may touch:
    cached rows get their bytes, new-token rows and the poison unit get the
    sentinel.  Small pools are sentinel-filled throughout."""
    ps = w.page_size
    if fill_all is None:
        fill_all = w.num_rows * ROW_BYTES <= (1 << 30)
    shape = (w.num_rows // ps, ps, HKV, D)
    if fill_all:
        kp = torch.full(shape, SENTINEL, dtype=torch.uint8, device=device)
        vp = torch.full(shape, SENTINEL, dtype=torch.uint8, device=device)
    else:
        kp = torch.empty(shape, dtype=torch.uint8, device=device)
        vp = torch.empty(shape, dtype=torch.uint8, device=device)
        kp[-1] = SENTINEL
        vp[-1] = SENTINEL
    for b in range(w.B):
        kb, vb = w.cache_values(b)
        idx = torch.from_numpy(w.pages[b]).to(device)
        kp[idx] = torch.from_numpy(_unit_blocks(w, b, kb)).to(device)
        vp[idx] = torch.from_numpy(_unit_blocks(w, b, vb)).to(device)
        del kb, vb
    return kp.view(w.num_rows, HKV, D), vp.view(w.num_rows, HKV, D)


class LogicalPool:
    """Row-indexable view of a huge pool holding only the rows of given requests.

    pool[rows] returns [n, 2, 64] bytes; rows that were never placed read as
    the sentinel.  Assigning pool[row] = bytes stores a row."""

    def __init__(self, w: Workload, requests, which: str, _values=None):
        ps = w.page_size
        rows, data = [], []
        for b in requests:
            kb, vb = _values[b] if _values is not None else w.cache_values(b)
            blk = _unit_blocks(w, b, kb if which == "k" else vb)
            r = (np.asarray(w.pages[b], dtype=np.int64)[:, None] * ps + np.arange(ps)[None, :])
            rows.append(r.reshape(-1))
            data.append(blk.reshape(-1, HKV, D))
        rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
        data = np.concatenate(data) if data else np.zeros((0, HKV, D), np.uint8)
        order = np.argsort(rows)
        self.rows = rows[order]
        self.data = data[order]

    @staticmethod
    def pair(w: Workload, requests) -> tuple["LogicalPool", "LogicalPool"]:
        """The K and V pools of the given requests, each request's cached
        bytes drawn once for both."""
        req = list(requests)
        vals = {b: w.cache_values(b) for b in req}
        return LogicalPool(w, req, "k", vals), LogicalPool(w, req, "v", vals)

    def _find(self, rows):
        rows = np.asarray(rows, dtype=np.int64)
        i = np.searchsorted(self.rows, rows)
        i = np.minimum(i, max(len(self.rows) - 1, 0))
        hit = (len(self.rows) > 0) & (self.rows[i] == rows) if len(self.rows) else np.zeros(rows.shape, bool)
        return i, hit

    def __getitem__(self, rows):
        i, hit = self._find(rows)
        out = np.full(np.shape(rows) + (HKV, D), SENTINEL, dtype=np.uint8)
        out[hit] = self.data[i[hit]]
        return out

    def __setitem__(self, row, value):
        i, hit = self._find(np.asarray([row]))
        if not hit[0]:
            raise KeyError(f"row {row} is not part of this logical pool")
        self.data[i[0]] = value


# --------------------------------------------------------------------------
# Output-projection inputs (plumbing): o [hidden, 1024] with N(0, 1/64^2)
# entries rounded to bf16 (the spread of a trained projection's weights), and
# standalone projection inputs a ~ N(0, 1/4) rounded to bf16.
# --------------------------------------------------------------------------

def oproj_weight(seed: int, hidden: int = 8192):
    import torch
    rng = np.random.default_rng([seed, 9, hidden])
    return torch.from_numpy(rng.standard_normal((hidden, 1024)).astype(np.float32) / 64.0
                            ).to(torch.bfloat16)


def oproj_input(seed: int, T: int):
    import torch
    rng = np.random.default_rng([seed, 10, T])
    return torch.from_numpy(rng.standard_normal((T, 1024)).astype(np.float32) * 0.5
                            ).to(torch.bfloat16)
