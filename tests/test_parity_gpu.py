"""GPU parity: the HIP step through the C ABI against the CPU oracle.

Bar: every written cache byte within 1 E4M3 ulp of the oracle's (v bytes exact
for power-of-two kv_scale); the oracle, attending to the GPU's own new
entries, matches the bf16 output within max-abs 2e-2 and mean-abs 2e-3.
"""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
from oracle import museattn_oracle as O
from paged_fp8_kv_amd import workloads as W

from gpu_common import (EPS, QS, ROPE_BASE, compare_out, full_check, gpu_new_bytes, log,
                        new_rows, oracle_prologue, run, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()   # raises if the HIP library is missing


def _untouched_rows_kept(w, d, host):
    """Every row other than the new tokens' rows still holds its old bytes."""
    rows = new_rows(w)
    for dev_pool, host_pool in ((d["k_cache"], host[0]), (d["v_cache"], host[1])):
        got = dev_pool.cpu().numpy()
        keep = np.ones(w.num_rows, bool)
        keep[rows] = False
        assert np.array_equal(got[keep], host_pool[keep]), "a row outside the new tokens changed"


# ------------------------------------------------ the workloads of record

@pytest.mark.parametrize("cid", ["0", "1", "3s", "3f"])
def test_config_parity(cid):
    w = W.config(cid)
    log(f"[config {cid}] {w.name} B={w.B} L={w.L} ctx={w.ctx.tolist()[:4]} ps={w.page_size}")
    host = W.build_pools_numpy(w)
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, host_pools=host)
    _untouched_rows_kept(w, d, host)


@pytest.mark.parametrize("cid", ["2", "4"])
def test_config_parity_full_size(cid):
    """Full-size pools and batch in the launch configuration the bench times
    (config 2: 32 requests over ~80 GB of pools; config 4: 16 requests, page
    size 64, kv_scale 1/64): every output element of every request against
    the oracle, every written byte within 1 ulp; then graph replays of the
    step, as the bench runs it, give the same bytes."""
    w = W.config(cid)
    log(f"[config {cid}] {w.name} B={w.B} pool rows={w.num_rows} checking all requests")
    d = upload(w)
    ws = torch.empty(P.workspace_bytes(w.B, w.L, w.max_seq_len, w.page_size, w.layer_kind),
                     dtype=torch.uint8, device="cuda:0")
    run(w, d, workspace=ws)
    torch.cuda.synchronize()
    full_check(w, d, requests=list(range(w.B)))
    # The launch configuration the benchmark times: several steps captured into
    # one HIP graph and replayed; every replay leaves the checked call's bytes.
    eager = d["out"].clone()
    log(f"[config {cid}] graph replays")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(w, d, workspace=ws)     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(4):
            run(w, d, workspace=ws)
    for i in range(3):
        d["out"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["out"], eager), f"replay {i} differs from the checked call"
        run(w, d, workspace=ws)     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(d["out"], eager)
    del g, d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cid,requests", [
    ("v32f", (0, 9, 22, 31)), ("v16f", (0, 15)), ("d16f", (0, 7, 15)),
    ("d32s", None), ("d16s", None), ("v32s", None), ("v16s", None)])
def test_batch_shapes_full_size(cid, requests):
    """The decode page's batch shapes (B 16 and 32, decode and verify blocks
    of 8, sliding and full layers, contexts U[60K, 100K]) at full size in the
    launch configuration the bench times: every written byte within 1 ulp,
    and the outputs of sampled requests (full layers) or of every request
    (sliding layers) against the oracle."""
    w = W.config(cid)
    reqs = list(range(w.B)) if requests is None else list(requests)
    log(f"[batch {cid}] {w.name} B={w.B} L={w.L} checking requests {reqs}")
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, requests=reqs)
    del d
    torch.cuda.empty_cache()


# ---------------------------------------------- edge cases and page's tests

EDGE = [
    # name, B, L, ctx, kind, page_size, kv_scale
    ("empty-context", 2, 1, 0, W.FULL, 1, 1.0),
    ("ctx10-sliding", 1, 1, 10, W.SLIDING, 64, 1.0),
    ("ctx2047-sliding-b3", 3, 1, 2047, W.SLIDING, 64, 1.0),
    ("b5-L8-sliding-ctx6000-spread", 5, 8, (3000, 6000), W.SLIDING, 1, 1.0),
    ("b4-full-ctx3000-p64", 4, 1, 3000, W.FULL, 64, 1.0),
    ("b4-L8-sliding-window-edges", 4, 8, (2038, 2058), W.SLIDING, 1, 1.0),
    ("b4-L8-full-ctx6000", 4, 8, 6000, W.FULL, 64, 1.0),
    ("b3-L8-sliding-kv1/64-p1", 3, 8, 4000, W.SLIDING, 1, 1.0 / 64),
    ("b2-full-kv1/64-p64", 2, 1, 9000, W.FULL, 64, 1.0 / 64),
    ("b2-L8-full-ctx20000-p64", 2, 8, 20000, W.FULL, 64, 1.0),
    ("b3-L2-full", 3, 2, (100, 700), W.FULL, 64, 1.0),
    ("b2-L3-sliding", 2, 3, (2500, 3000), W.SLIDING, 1, 1.0),
    ("b2-L5-full", 2, 5, (900, 1300), W.FULL, 1, 1.0),
    ("b2-L7-sliding", 2, 7, (3000, 3100), W.SLIDING, 64, 1.0),
    ("b33-full-ctx25000-spread", 33, 1, (12500, 25000), W.FULL, 1, 1.0),
    ("b2-full-kv0.3", 2, 1, 500, W.FULL, 1, 0.3),
    ("b1-L8-ragged-tail", 1, 8, 4125, W.FULL, 1, 1.0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_parity(case):
    name, B, L, ctx, kind, ps, kv = case
    w = W.make(name, 77, B, L, ctx, kind, ps, kv)
    log(f"[edge] {name} ctx={w.ctx.tolist()[:6]} work-groups={P.work_groups(B, L, w.max_seq_len, kind)}")
    host = W.build_pools_numpy(w)
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, host_pools=host)
    _untouched_rows_kept(w, d, host)


# The page's gate tests that the edge cases above do not already cover
# (section "Correctness" gives the distributions; "heads dp" shapes run at this
# shard's head count; "spread mixed" draws each context from [ctx/2, ctx]).
GATE = [
    # name, B, L, ctx, kind, page_size, kv_scale, dist
    ("gate-b8-full-ctx8192-spread", 8, 1, (4096, 8192), W.FULL, 1, 1.0, "soft"),
    ("gate-b2-L8-full-ctx100000-p1", 2, 8, 100000, W.FULL, 1, 1.0, "soft"),
    ("gate-b4-sliding-ctx6000-edges-p1", 4, 1, 6000, W.SLIDING, 1, 1.0, "edges"),
    ("gate-b4-L8-full-ctx6000-edges", 4, 8, 6000, W.FULL, 64, 1.0, "edges"),
    ("gate-b4-full-ctx80000-spread-soft", 4, 1, (40000, 80000), W.FULL, 64, 1.0, "soft"),
    ("gate-b4-L8-sliding-ctx6000-soft-p1", 4, 8, 6000, W.SLIDING, 1, 1.0, "soft"),
    ("gate-b4-full-ctx80000-spread-coherent-p1", 4, 1, (40000, 80000), W.FULL, 1, 1.0, "coherent"),
    ("gate-b2-L8-full-ctx20000-coherent", 2, 8, 20000, W.FULL, 64, 1.0, "coherent"),
    ("b3-L8-sliding-ctx5000-coherent", 3, 8, 5000, W.SLIDING, 1, 1.0, "coherent"),
    ("b2-L3-sliding-ctx3000-edges-kv1/64", 2, 3, 3000, W.SLIDING, 64, 1.0 / 64, "edges"),
]


@pytest.mark.parametrize("case", GATE, ids=[c[0] for c in GATE])
def test_gate_parity(case):
    name, B, L, ctx, kind, ps, kv, dist = case
    w = W.make(name, 88, B, L, ctx, kind, ps, kv, dist=dist)
    log(f"[gate] {name} ctx={w.ctx.tolist()[:4]} dist={dist}")
    host = W.build_pools_numpy(w)
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, host_pools=host)
    _untouched_rows_kept(w, d, host)


@pytest.mark.slow
def test_million_key_verify_block():
    """A full layer over 1,048,576 cached keys with an 8-token block."""
    w = W.make("ctx1M-L8-full", 91, 1, 8, 1048576, W.FULL, 1, 1.0)
    log(f"[edge] {w.name}")
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, requests=[0])


def test_maximum_batch():
    """1,024 requests, the most one call takes: the plan's prefix sums hold two
    units per thread, and work-group shares cross many request boundaries."""
    for L, kind in ((1, W.FULL), (2, W.SLIDING)):
        w = W.make(f"max-batch-L{L}", 41, 1024, L, (1, 300), kind, 1, 1.0)
        log(f"[edge] {w.name} work-groups={P.work_groups(w.B, L, w.max_seq_len, kind)}")
        host = W.build_pools_numpy(w)
        d = upload(w)
        run(w, d)
        torch.cuda.synchronize()
        full_check(w, d, host_pools=host)
        del d


# ----------------------------------------------------------- properties

def test_partition_invariance_and_determinism():
    """The work-group count changes only the summation order; one, a prime
    number, and more work-groups than chunks (some then idle) all agree."""
    w = W.make("partition", 5, 3, 1, (3000, 9000), W.FULL, 1, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    outs = []
    for g in (1, 7, 64, 509, 4096, 0):
        log(f"[partition] work_groups={g}")
        run(w, d, work_groups=g)
        outs.append(d["out"].clone())
    torch.cuda.synchronize()
    full_check(w, d, host_pools=host)
    ref = outs[-1].float()
    for o in outs[:-1]:
        assert (o.float() - ref).abs().max().item() <= 1.6e-2
    run(w, d)
    assert torch.equal(d["out"], outs[-1]), "two identical calls differ"


def test_verify_partition_invariance():
    w = W.make("vpartition", 6, 2, 8, (2500, 4000), W.SLIDING, 1, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    outs = []
    for g in (1, 3, 100, 1000, 0):
        run(w, d, work_groups=g)
        outs.append(d["out"].clone())
    torch.cuda.synchronize()
    full_check(w, d, host_pools=host)
    for o in outs[:-1]:
        assert (o.float() - outs[-1].float()).abs().max().item() <= 1.6e-2


def test_verify_full_layer_partition_invariance():
    """Full-layer verify blocks of 9K-12K keys: with one or five work-groups
    a segment spans several 4096-key LDS fills of row ids, so the staging
    ring crosses fill boundaries; with 64 the segments are short.  Every
    count agrees with the oracle and with the default partition."""
    w = W.make("vfull-partition", 8, 2, 8, (9000, 12000), W.FULL, 1, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    outs = []
    for g in (1, 5, 64, 0):
        log(f"[vfull-partition] work_groups={g}")
        run(w, d, work_groups=g)
        torch.cuda.synchronize()
        full_check(w, d, host_pools=host)
        outs.append(d["out"].clone())
    for o in outs[:-1]:
        assert (o.float() - outs[-1].float()).abs().max().item() <= 1.6e-2


@pytest.mark.parametrize("L,kind", [(1, W.FULL), (1, W.SLIDING), (8, W.FULL)],
                         ids=["decode-full", "decode-sliding", "verify-L8-full"])
def test_one_request_partition_invariance(L, kind):
    """One request: with at most 48 candidate slots (work-groups 0 ..
    min(work-groups, chunks + costs) - 1) its merge loads them all with its
    plan and keeps those the plan names; with more it reads the plan first.
    Work-group counts that give 1 and 3 candidates per slot lane (1, 5, 16;
    17, 48) and counts past the switch (49 to 300 and the default) all agree
    with the oracle and with each other."""
    w = W.make(f"one-request-L{L}", 9 + L + kind, 1, L, 20000, kind, 1, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    outs = []
    for g in (1, 5, 16, 17, 48, 49, 200, 256, 300, 0):
        log(f"[one-request L={L} kind={kind}] work_groups={g}")
        run(w, d, work_groups=g)
        torch.cuda.synchronize()
        full_check(w, d, host_pools=host)
        outs.append(d["out"].clone())
    for o in outs[:-1]:
        assert (o.float() - outs[-1].float()).abs().max().item() <= 1.6e-2
    run(w, d)
    assert torch.equal(d["out"], outs[-1]), "two identical calls differ"


@pytest.mark.parametrize("L,B,ctx,ps,msl", [
    (1, 8, (3000, 9000), 1, 300000), (1, 8, (3000, 9000), 64, 300000),
    (1, 8, (3000, 9000), 64, 200000), (8, 1, 5000, 1, 300000), (8, 2, 4000, 64, 300000),
    (8, 8, 1500, 1, 300000)],
    ids=["decode-ps1-586MB", "decode-ps64-586MB", "decode-ps64-391MB", "verify-ps1-73MB",
         "verify-ps64-146MB", "verify-ps1-586MB"])
def test_nontemporal_paths_match(L, B, ctx, ps, msl):
    """The paths chosen by the step's size: a decode step that may read more
    than 512 MB of rows (B x max_seq_len x 256 B) loads V and stores its
    partials non-temporally; at page size 64, from 256 MB, it loads V
    non-temporally with ordinary partial stores; a verify block from 4 MB
    stores its partials non-temporally, and above 512 MB also reads its rows
    into the ring non-temporally.  Declaring a larger max_seq_len for
    small requests selects those paths at a size the oracle checks: each
    gives the bytes of the ordinary path (same arithmetic in the same order)
    over several partitions, and meets the oracle."""
    w = W.make(f"nt-L{L}-ps{ps}", 40 + ps + L, B, L, ctx, W.FULL, ps, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    nt_min = (4 if L > 1 else 256 if ps == 64 else 512) << 20
    assert w.B * msl * 256 > nt_min and w.B * w.max_seq_len * 256 < nt_min
    stride = -(-msl // ps)
    table = torch.full((w.B, stride), -1, dtype=torch.int32)
    table[:, :w.table_stride] = torch.from_numpy(w.table)
    table = table.cuda()
    for g in (0, 7, 64):
        log(f"[nt L={L} ps={ps} max_seq_len={msl}] work_groups={g}")
        run(w, d, work_groups=g)
        torch.cuda.synchronize()
        ordinary = d["out"].clone()
        P.attn_step(d["qkv"], d["positions"], table, d["seq_lens"], d["k_cache"], d["v_cache"],
                    w.kv_scale, w.page_size, w.layer_kind, d["out"], q_norm_w=d["w_q"],
                    k_norm_w=d["w_k"], o_norm_w=d["w_o"], max_seq_len=msl, eps=EPS, q_scale=QS,
                    rope_base=ROPE_BASE, work_groups=g)
        torch.cuda.synchronize()
        assert torch.equal(d["out"], ordinary), f"work_groups={g}: the two load paths differ"
    full_check(w, d, host_pools=host)


def test_many_requests_sharing_work_groups():
    """More requests than chunks per work-group: shares cross several request
    boundaries, so segments, partial slots and the last-contributor merge are
    all exercised (and some requests have a single chunk)."""
    w = W.make("many-short", 21, 300, 1, (1, 90), W.FULL, 64, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    for g in (0, 97):
        run(w, d, work_groups=g)
        torch.cuda.synchronize()
        full_check(w, d, host_pools=host)


@pytest.mark.parametrize("L,kind", [(8, W.FULL), (5, W.SLIDING), (40, W.FULL)],
                         ids=["verify-full", "verify-sliding", "prefill"])
def test_causal_in_block(L, kind):
    """Changing the last block token's row (its q, k, v and gate) leaves every
    earlier token's output bitwise unchanged: none of them sees its key."""
    w = W.make(f"causal-L{L}", 17, 3, L, (1500, 3000), kind, 1, 1.0)
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    before = d["out"].clone()
    g = torch.Generator().manual_seed(5)
    last = torch.arange(w.B) * L + (L - 1)
    d["qkv"][last] = torch.randn(w.B, d["qkv"].shape[1], generator=g).to(torch.bfloat16).cuda()
    run(w, d)
    torch.cuda.synchronize()
    assert torch.equal(d["out"][:, :L - 1], before[:, :L - 1])
    assert not torch.equal(d["out"][:, L - 1], before[:, L - 1])


@pytest.mark.parametrize("L", [1, 8], ids=["decode", "verify"])
def test_requests_are_independent(L):
    """Request 2's inputs and cached rows changed: the other requests' outputs
    stay bitwise the same (work-group shares that span two requests keep
    separate states per request)."""
    w = W.make(f"indep-L{L}", 18, 4, L, (3000, 6000), W.FULL, 1, 1.0)
    d = upload(w)
    run(w, d, work_groups=7)   # shares cross request boundaries
    torch.cuda.synchronize()
    before = d["out"].clone()
    g = torch.Generator().manual_seed(6)
    d["qkv"][2 * L:3 * L] = torch.randn(L, d["qkv"].shape[1], generator=g).to(torch.bfloat16).cuda()
    rows = torch.from_numpy(w.table[2, :int(w.ctx[2])].astype(np.int64)).cuda()
    d["k_cache"][rows] = torch.randint(0, 0x7e, (rows.numel(), 2, 64), generator=g,
                                       dtype=torch.uint8).cuda()
    run(w, d, work_groups=7)
    torch.cuda.synchronize()
    keep = [0, 1, 3]
    assert torch.equal(d["out"][keep], before[keep])
    assert not torch.equal(d["out"][2], before[2])


def test_page_size_does_not_change_the_result():
    outs = []
    for ps in (1, 64):
        w = W.make("ps", 12, 4, 8, (700, 1500), W.FULL, ps, 1.0)
        d = upload(w)
        run(w, d)
        outs.append(d["out"].clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_value_encoder_exhaustive_over_bf16():
    """v goes to the cache unnormed, so every finite bf16 value (and +-inf) is
    fed to the fp8 encoder; with kv_scale 1 the bytes must equal the oracle's
    exactly (ties to even, subnormals, saturation at +-448)."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).copy()
    vals[np.isnan(vals)] = 1.0
    w = W.make("v-encoder", 3, 64, 8, 4, W.FULL, 1, 1.0)
    qkv = w.qkv.clone()
    qkv[:, 1152:1280] = torch.from_numpy(vals).to(torch.bfloat16).view(512, 128)
    w.qkv = qkv
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    _, vb_gpu = gpu_new_bytes(w, d)
    _, _, vb, _ = oracle_prologue(w)
    assert np.array_equal(vb_gpu, vb)


@pytest.mark.parametrize("L", [1, 8, 40], ids=["decode", "verify", "prefill"])
def test_other_norm_and_rope_parameters(L):
    """eps, q_scale and rope_base reach every kernel: eps 1e-5, q_scale 1 and
    rope base 500,000 on a sliding layer, 64-token pages, kv_scale 1/64."""
    eps, qs, base = float(np.float32(1e-5)), 1.0, 500000.0
    w = W.make(f"params-L{L}", 32, 2, L, (2500, 4000), W.SLIDING, 64, 1.0 / 64)
    host = W.build_pools_numpy(w)
    d = upload(w)
    P.attn_step(d["qkv"], d["positions"], d["table"], d["seq_lens"], d["k_cache"], d["v_cache"],
                w.kv_scale, w.page_size, w.layer_kind, d["out"],
                q_norm_w=d["w_q"], k_norm_w=d["w_k"], o_norm_w=d["w_o"],
                max_seq_len=w.max_seq_len, eps=eps, q_scale=qs, rope_base=base)
    torch.cuda.synchronize()
    kb_gpu, vb_gpu = gpu_new_bytes(w, d)
    _, kb, vb, _ = O.prologue(w.qkv.float().numpy(), w.positions, w.w_q, w.w_k, eps=eps,
                              q_scale=qs, rope=True, rope_base=base, kv_scale=w.kv_scale)
    assert np.abs(O.e4m3_ordinal(kb_gpu) - O.e4m3_ordinal(kb)).max() <= 1
    assert np.array_equal(vb_gpu, vb)
    want, _, _ = O.attn_step(w.qkv.float().numpy(), w.positions, w.table, host[0].copy(),
                             host[1].copy(), B=w.B, L=w.L, page_size=w.page_size,
                             layer_kind=w.layer_kind, kv_scale=w.kv_scale, w_q=w.w_q, w_k=w.w_k,
                             w_o=w.w_o, eps=eps, q_scale=qs, rope_base=base,
                             new_rows=(kb_gpu, vb_gpu))
    compare_out(d["out"].float().cpu().numpy(), want, w.name)


@pytest.mark.parametrize("L", [1, 8, 40], ids=["decode", "verify", "prefill"])
def test_q_beyond_half_precision_range(L):
    """q_scale 1e6 puts |q| * log2(e)/8 far past 65504, the largest fp16
    value the block path's q operand can hold: such a column is held as
    q * 2^-e and its products are scaled back by 2^e.  The softmax is then a
    hard argmax (scores of order 1e7 in log2 units), so the output of a
    (token, head) is the gated norm of its best key's v.  Columns whose two
    best keys lie closer than the fp16 rounding of q can move (2^14 log2
    units) are left out: either key is a correct answer there."""
    qs = 1.0e6
    w = W.make(f"big-q-L{L}", 31, 2, L, 300, W.FULL, 1, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    P.attn_step(d["qkv"], d["positions"], d["table"], d["seq_lens"], d["k_cache"], d["v_cache"],
                w.kv_scale, w.page_size, w.layer_kind, d["out"],
                q_norm_w=d["w_q"], k_norm_w=d["w_k"], o_norm_w=d["w_o"],
                max_seq_len=w.max_seq_len, eps=EPS, q_scale=qs, rope_base=10000.0)
    torch.cuda.synchronize()
    kb_gpu, vb_gpu = gpu_new_bytes(w, d)
    kp, vp = host[0].copy(), host[1].copy()
    want, _, _ = O.attn_step(w.qkv.float().numpy(), w.positions, w.table, kp, vp, B=w.B, L=w.L,
                             page_size=1, layer_kind=W.FULL, kv_scale=1.0, w_q=w.w_q, w_k=w.w_k,
                             w_o=w.w_o, eps=EPS, q_scale=qs, new_rows=(kb_gpu, vb_gpu))
    # the gap between each column's two best scores (log2 units), from the
    # pools the oracle attended to
    q = O.prologue(w.qkv.float().numpy(), w.positions, w.w_q, w.w_k, eps=EPS, q_scale=qs,
                   rope=False, rope_base=10000.0, kv_scale=1.0)[0]
    keep = np.zeros((w.B, w.L, 16), bool)
    for b in range(w.B):
        for jt in range(w.L):
            p = int(w.positions[b * w.L + jt])
            kd = O.e4m3_decode(kp[O.cache_row(w.table, b, np.arange(p + 1), 1)])
            for h in range(16):
                sc = np.sort(kd[:, h // 8, :] @ q[b * w.L + jt, h] / 8.0 * np.log2(np.e))
                keep[b, jt, h] = sc[-1] - sc[-2] > 2.0 ** 14
    assert keep.mean() > 0.9
    got = d["out"].float().cpu().numpy().reshape(w.B, w.L, 16, 64)[keep]
    compare_out(got, want.reshape(w.B, w.L, 16, 64)[keep], f"{w.name} ({int(keep.sum())} columns)")


@pytest.mark.parametrize("L,kind", [(1, W.FULL), (8, W.SLIDING), (40, W.FULL)],
                         ids=["decode", "verify", "prefill"])
def test_graph_capture_replays_match_eager(L, kind):
    """The step captured into a HIP graph (as a decode loop replays it) gives
    the eager call's bytes on every replay, with eager calls in between."""
    w = W.make(f"graph-L{L}", 8, 4, L, (2000, 5000), kind, 1, 1.0)
    d = upload(w)
    ws = torch.empty(P.workspace_bytes(w.B, w.L, w.max_seq_len, w.page_size, w.layer_kind),
                     dtype=torch.uint8, device="cuda:0")
    run(w, d, workspace=ws)
    torch.cuda.synchronize()
    eager = d["out"].clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(w, d, workspace=ws)     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run(w, d, workspace=ws)
    for i in range(3):
        d["out"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["out"], eager), f"replay {i} differs from the eager call"
        run(w, d, workspace=ws)     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(d["out"], eager)
