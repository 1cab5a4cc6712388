"""Helpers of the GPU parity tests: upload a workload, run the HIP step through
the C ABI, and check it against the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_fp8_kv_amd as P
from oracle import museattn_oracle as O
from paged_fp8_kv_amd import workloads as W

EPS = float(np.float32(1e-6))
QS = float(np.float32(5.473))
ROPE_BASE = 10000.0
# Output bar: bf16 output vs the float64 oracle (the oracle attends to the
# GPU's own new cache entries, as the page's correctness section does).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def upload(w: W.Workload, dev="cuda:0", fill_all=None) -> dict:
    kp, vp = W.build_pools_device(w, dev, fill_all)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    return dict(qkv=w.qkv.to(dev), positions=f(w.positions), table=f(w.table),
                seq_lens=f(w.seq_lens), w_q=f(w.w_q), w_k=f(w.w_k), w_o=f(w.w_o),
                k_cache=kp, v_cache=vp,
                out=torch.empty(w.B, w.L, 1024, dtype=torch.bfloat16, device=dev))


def run(w: W.Workload, d: dict, work_groups=0, stream=None, workspace=None):
    P.attn_step(d["qkv"], d["positions"], d["table"], d["seq_lens"], d["k_cache"], d["v_cache"],
                w.kv_scale, w.page_size, w.layer_kind, d["out"], stream,
                q_norm_w=d["w_q"], k_norm_w=d["w_k"], o_norm_w=d["w_o"],
                max_seq_len=w.max_seq_len, workspace=workspace, eps=EPS, q_scale=QS,
                rope_base=ROPE_BASE, work_groups=work_groups)
    return d["out"]


def new_rows(w: W.Workload) -> np.ndarray:
    return np.array([int(O.cache_row(w.table, t // w.L, int(w.positions[t]), w.page_size))
                     for t in range(w.T)], dtype=np.int64)


def gpu_new_bytes(w: W.Workload, d: dict):
    rows = torch.from_numpy(new_rows(w)).to(d["k_cache"].device)
    return d["k_cache"][rows].cpu().numpy(), d["v_cache"][rows].cpu().numpy()


def oracle_prologue(w: W.Workload):
    return O.prologue(w.qkv.float().numpy(), w.positions, w.w_q, w.w_k, eps=EPS, q_scale=QS,
                      rope=w.layer_kind == W.SLIDING, rope_base=ROPE_BASE, kv_scale=w.kv_scale)


def check_bytes(w: W.Workload, kb_gpu, vb_gpu):
    """Written entries within 1 fp8 ulp of the oracle's; v exact when kv_scale is a
    power of two (v / kv_scale is then exact on both sides)."""
    _, kb, vb, _ = oracle_prologue(w)
    dk = np.abs(O.e4m3_ordinal(kb_gpu) - O.e4m3_ordinal(kb))
    dv = np.abs(O.e4m3_ordinal(vb_gpu) - O.e4m3_ordinal(vb))
    assert dk.max() <= 1, f"k bytes off by {dk.max()} ulp"
    assert dv.max() <= 1, f"v bytes off by {dv.max()} ulp"
    if np.log2(w.kv_scale).is_integer():
        assert dv.max() == 0, "v bytes must be exact for power-of-two kv_scale"
    return float((dk == 0).mean())


def oracle_out(w: W.Workload, kb_gpu, vb_gpu, pools=None, tokens=None):
    """Oracle output attending to the GPU's new entries.  pools: host pools
    (numpy) or None for a logical pool of w's requests."""
    if pools is None:
        kp, vp = W.LogicalPool.pair(w, range(w.B))
    else:
        kp, vp = pools[0].copy(), pools[1].copy()
    out, _, _ = O.attn_step(w.qkv.float().numpy(), w.positions, w.table, kp, vp, B=w.B, L=w.L,
                            page_size=w.page_size, layer_kind=w.layer_kind,
                            kv_scale=w.kv_scale, w_q=w.w_q, w_k=w.w_k, w_o=w.w_o, eps=EPS,
                            q_scale=QS, rope_base=ROPE_BASE, new_rows=(kb_gpu, vb_gpu),
                            tokens=tokens)
    return out


def compare_out(got: np.ndarray, want: np.ndarray, label: str):
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    err = np.abs(got.astype(np.float64) - want)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {label}: max-abs {mx:.3e}  mean-abs {mean:.3e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{label}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


def full_check(w: W.Workload, d: dict, requests=None, host_pools=None, tokens=None):
    """Bytes and output of a finished GPU step against the oracle.  requests:
    subset of requests whose outputs the oracle recomputes (None = all);
    tokens: block-token indices compared (None = all)."""
    kb_gpu, vb_gpu = gpu_new_bytes(w, d)
    exact = check_bytes(w, kb_gpu, vb_gpu)
    got = d["out"].float().cpu().numpy()
    if requests is None:
        want = oracle_out(w, kb_gpu, vb_gpu, host_pools, tokens)
        if tokens is not None:
            got, want = got[:, tokens], want[:, tokens]
        label = f"{w.name} (exact k bytes {exact:.4f})" + ("" if tokens is None else f" tokens {list(tokens)[:6]}..")
        return compare_out(got, want, label)
    sub = w.subset(requests)
    sel = np.array([[b * w.L + j for j in range(w.L)] for b in requests]).reshape(-1)
    want = oracle_out(sub, kb_gpu[sel], vb_gpu[sel], None)
    return compare_out(got[list(requests)], want, f"{w.name} requests {list(requests)}")
