"""GPU parity of the attention output projection (task page "Whole decoder
layer", section "What to compute": y = out @ o^T), through the C ABI.

* museattn_oproj alone on bf16 inputs: the oracle's float64 product of the
  same bf16 values; the GPU differs by its fp32 sums and the bf16 rounding of
  y, so each element must lie within one bf16 rounding (2^-8 relative) plus
  1e-5 of the sum of |a_k o_nk| (fp32 accumulation over 1024 terms).
* the step followed by the projection: y against the oracle's step output
  (float64, attending to the GPU's own new entries) times o^T, at the step's
  bar (max-abs 2e-2, mean-abs 2e-3).
"""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
from oracle import museattn_oracle as O
from paged_fp8_kv_amd import workloads as W

from gpu_common import (EPS, MAX_ABS, MEAN_ABS, QS, ROPE_BASE, compare_out, gpu_new_bytes, log,
                        oracle_out, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()


@pytest.mark.parametrize("T,hidden", [(1, 64), (7, 8192), (32, 8192), (33, 1088), (63, 8192),
                                      (64, 8192), (65, 64), (100, 2048), (129, 1088), (159, 1088),
                                      (256, 8192), (384, 8192), (753, 8192), (1024, 64),
                                      (1000, 1088), (1024, 8192), (2048, 8192), (3012, 8192),
                                      (13100, 1088)])
def test_oproj_alone(T, hidden):
    """Up to 63 tokens the register kernel runs (32 rows of o per work-group,
    64-token passes: T 7, 33 and 63 end inside a pass); from 64 on the
    LDS-tiled GEMM (T 63 and 64 sit on either side of the switch).  The
    GEMM's tile shapes: 128 x 64 (T 64 to 256 at hidden 8192; T 1000 and
    hidden 1088, whose last feature and token tiles are partial; hidden 64,
    half a tile), 128 x 128 (T 384), 128 x 192 (T 753 and 3012; T 13100 with
    hidden 1088: partial tiles on both axes), 256 x 128 (T 1024) and 256 x
    256 (T 2048)."""
    a = W.oproj_input(70 + T, T)
    o = W.oproj_weight(71, hidden)
    y = torch.empty(T, hidden, dtype=torch.bfloat16, device="cuda")
    P.oproj(a.cuda(), o.cuda(), y)
    torch.cuda.synchronize()
    af, of = a.double().numpy(), o.double().numpy()
    want = O.oproj(af, of)
    bound = np.abs(want) * 2.0 ** -8 + 1e-5 * (np.abs(af) @ np.abs(of).T) + 1e-30
    err = np.abs(y.double().cpu().numpy() - want)
    log(f"  oproj T={T} hidden={hidden}: max err/bound {float((err / bound).max()):.3f}")
    assert (err <= bound).all()


def test_oproj_rejects_bad_arguments():
    a = torch.zeros(4, 1024, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(24, 1024, dtype=torch.bfloat16, device="cuda")   # hidden not a multiple of 64
    y = torch.zeros(4, 24, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P.MuseAttnError) as e:
        P.oproj(a, o, y)
    assert e.value.status == -8


STEP_CASES = [
    # name, config builder
    ("decode-b32-full", lambda: W.make("op-decode-b32-full", 80, 32, 1, (3000, 6000), W.FULL, 1, 1.0)),
    ("verify-b4-L8-sliding", lambda: W.make("op-verify-b4-sliding", 81, 4, 8, (2500, 4000),
                                             W.SLIDING, 64, 1.0 / 64)),
    ("prefill-b1-L40-full", lambda: W.make("op-prefill-b1-L40", 82, 1, 40, 700, W.FULL, 1, 1.0)),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_step_then_oproj(case):
    name, build = case
    w = build()
    d = upload(w)
    o = W.oproj_weight(83, 8192).cuda()
    y = torch.empty(w.T, 8192, dtype=torch.bfloat16, device="cuda")
    P.attn_step(d["qkv"], d["positions"], d["table"], d["seq_lens"], d["k_cache"], d["v_cache"],
                w.kv_scale, w.page_size, w.layer_kind, d["out"], q_norm_w=d["w_q"],
                k_norm_w=d["w_k"], o_norm_w=d["w_o"], max_seq_len=w.max_seq_len, eps=EPS,
                q_scale=QS, rope_base=ROPE_BASE, o_weight=o, y=y)
    torch.cuda.synchronize()
    kb, vb = gpu_new_bytes(w, d)
    out = oracle_out(w, kb, vb).reshape(w.T, 1024)
    want = O.oproj(out, o.double().cpu().numpy())
    compare_out(d["out"].float().cpu().numpy().reshape(w.T, 1024), out, f"{name} out")
    compare_out(y.float().cpu().numpy(), want, f"{name} y")


@pytest.mark.parametrize("T", [32, 256, 753, 2048])
def test_oproj_graph_replays_match_eager(T):
    """The projection captured into a HIP graph on its first call of the shape
    (the library keeps nothing between calls, so nothing has to be set up
    first) -- the register kernel at 32 tokens, the GEMM at 256, 753 and 2048 --
    gives the eager call's bytes on every replay, with eager calls in between."""
    a = W.oproj_input(90 + T, T).cuda()
    o = W.oproj_weight(91, 8192).cuda()
    y = torch.empty(T, 8192, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.oproj(a, o, y)
    y.zero_()
    P.oproj(a, o, y)   # the eager result
    torch.cuda.synchronize()
    eager = y.clone()
    for i in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {i} differs from the eager call"
        P.oproj(a, o, y)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, eager)


FUSED_CASES = [
    # name, workload builder, hidden: every merge kind the step can end with,
    # both projection kernels and hidden sizes from 64 to 16,384.
    ("decode-b1-long-h8192", lambda: W.make("opf-decode-b1", 84, 1, 1, 20000, W.FULL, 1, 1.0), 8192),
    ("decode-b3-h64", lambda: W.make("opf-decode-b3", 85, 3, 1, (1, 900), W.FULL, 64, 1.0), 64),
    ("verify-b24-L2-sliding-h1088", lambda: W.make("opf-verify-b24", 86, 24, 2, (2100, 2600),
                                                   W.SLIDING, 1, 1.0), 1088),
    ("verify-b9-L7-full-h8192", lambda: W.make("opf-verify-b9", 87, 9, 7, (500, 1500), W.FULL, 1,
                                               1.0), 8192),
    ("verify-b8-L8-full-h8192", lambda: W.make("opf-verify-b8", 90, 8, 8, (500, 1500), W.FULL, 1,
                                               1.0), 8192),
    ("prefill-b5-L13-h8192", lambda: W.make("opf-prefill-b5", 88, 5, 13, (100, 400), W.FULL, 1,
                                            1.0), 8192),
    ("decode-b16-h16384", lambda: W.make("opf-decode-b16", 89, 16, 1, (300, 700), W.FULL, 1, 1.0),
     16384),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_step_projection_matches_projection_alone(case):
    """museattn_attn_step_oproj's y has the bytes museattn_oproj gives on the
    step's output, after the per-(token, head) merge with short (B 3, 9, 16)
    and long (B 1, 20,000 keys) slot lists and after the per-token merge (B 24,
    L 2; prefill), on the register kernel (63 tokens nearly fill its one pass)
    and on the GEMM (64, 65 tokens).  The step's output itself meets the
    oracle's bar."""
    name, build, hidden = case
    w = build()
    d = upload(w)
    o = W.oproj_weight(92, hidden).cuda()
    y = torch.full((w.T, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    log(f"[{name}] T={w.T} hidden={hidden}")
    P.attn_step(d["qkv"], d["positions"], d["table"], d["seq_lens"], d["k_cache"], d["v_cache"],
                w.kv_scale, w.page_size, w.layer_kind, d["out"], q_norm_w=d["w_q"],
                k_norm_w=d["w_k"], o_norm_w=d["w_o"], max_seq_len=w.max_seq_len, eps=EPS,
                q_scale=QS, rope_base=ROPE_BASE, o_weight=o, y=y)
    alone = torch.empty_like(y)
    P.oproj(d["out"].reshape(w.T, 1024), o, alone)
    torch.cuda.synchronize()
    assert torch.equal(y, alone), f"{name}: y differs from the projection of the step's output"
    kb, vb = gpu_new_bytes(w, d)
    out = oracle_out(w, kb, vb).reshape(w.T, 1024)
    compare_out(d["out"].float().cpu().numpy().reshape(w.T, 1024), out, f"{name} out")


def test_step_with_projection_graph_replays_match_eager():
    """Decode B 32 followed by the projection, captured into a HIP graph on
    the first call: every replay gives the eager call's y, with eager steps
    in between."""
    w = W.make("opf-graph", 93, 32, 1, (2000, 4000), W.FULL, 1, 1.0)
    d = upload(w)
    o = W.oproj_weight(94, 8192).cuda()
    y = torch.empty(w.T, 8192, dtype=torch.bfloat16, device="cuda")

    def step():
        P.attn_step(d["qkv"], d["positions"], d["table"], d["seq_lens"], d["k_cache"],
                    d["v_cache"], w.kv_scale, w.page_size, w.layer_kind, d["out"],
                    q_norm_w=d["w_q"], k_norm_w=d["w_k"], o_norm_w=d["w_o"],
                    max_seq_len=w.max_seq_len, eps=EPS, q_scale=QS, rope_base=ROPE_BASE,
                    o_weight=o, y=y)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {i} differs from the eager step"
        step()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
