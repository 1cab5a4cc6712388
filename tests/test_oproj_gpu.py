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


@pytest.mark.parametrize("T,hidden", [(1, 64), (7, 8192), (32, 8192), (33, 1088), (64, 8192),
                                      (65, 64), (100, 2048), (129, 1088), (159, 1088),
                                      (160, 8192), (256, 8192), (753, 8192), (1024, 64)])
def test_oproj_alone(T, hidden):
    """Up to 159 tokens the library's kernel runs (32 rows of o per work-group,
    64-token passes: T 33, 65, 100, 129 and 159 end inside a pass); from 160 on
    the hipBLASLt GEMM (T 159 and 160 sit on either side of the switch, hidden
    64 is its smallest shape)."""
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


@pytest.mark.parametrize("T", [32, 753])
def test_oproj_graph_replays_match_eager(T):
    """The projection captured into a HIP graph -- the library's kernel at 32
    tokens, the hipBLASLt GEMM at 753 -- gives the eager call's bytes on every
    replay, with eager calls in between."""
    a = W.oproj_input(90 + T, T).cuda()
    o = W.oproj_weight(91, 8192).cuda()
    y = torch.empty(T, 8192, dtype=torch.bfloat16, device="cuda")
    P.oproj(a, o, y)   # first call of the shape: makes the plan outside the capture
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        P.oproj(a, o, y)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        P.oproj(a, o, y)
    for i in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {i} differs from the eager call"
        P.oproj(a, o, y)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
