"""GPU parity of long blocks (prefill, L > 8): the HIP step through the C ABI
against the CPU oracle, same bar as the decode and verify tests.

Shapes: the prefill task page's gate tests (section "Shapes"; its one test
without "page 1" is read as the 64-token-page one) and scored shapes, the
latter with the oracle on sampled block tokens.
"""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
from paged_fp8_kv_amd import workloads as W

from gpu_common import full_check, log, new_rows, run, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()   # raises if the HIP library is missing


def _untouched_rows_kept(w, d, host):
    rows = new_rows(w)
    for dev_pool, host_pool in ((d["k_cache"], host[0]), (d["v_cache"], host[1])):
        got = dev_pool.cpu().numpy()
        keep = np.ones(w.num_rows, bool)
        keep[rows] = False
        assert np.array_equal(got[keep], host_pool[keep]), "a row outside the new tokens changed"


GATE = [
    # name, B, L, ctx, kind, page_size, kv_scale, dist
    ("pf-b1-ctx0-sliding-L300", 1, 300, 0, W.SLIDING, 1, 1.0, "soft"),
    ("pf-b1-ctx3000-full-L753", 1, 753, 3000, W.FULL, 1, 1.0, "soft"),
    ("pf-b2-ctx2500-sliding-L753", 2, 753, 2500, W.SLIDING, 1, 1.0, "soft"),
    ("pf-b3-ctx5000-full-L200-outliers-p64", 3, 200, 5000, W.FULL, 64, 1.0, "outliers"),
    ("pf-b1-ctx4096-sliding-L4096", 1, 4096, 4096, W.SLIDING, 1, 1.0, "soft"),
    # group boundaries, spread contexts, kv_scale 1/64, window edges
    ("pf-b3-L9-sliding", 3, 9, 1000, W.SLIDING, 1, 1.0, "soft"),
    ("pf-b2-L17-full-p64", 2, 17, 3000, W.FULL, 64, 1.0, "soft"),
    ("pf-b2-L33-sliding-window-edges", 2, 33, (2030, 2070), W.SLIDING, 1, 1.0, "edges"),
    ("pf-b4-L100-full-spread-kv1/64-p64", 4, 100, (1500, 3000), W.FULL, 64, 1.0 / 64, "soft"),
    ("pf-b2-L64-full-coherent", 2, 64, 6000, W.FULL, 1, 1.0, "coherent"),
]


@pytest.mark.parametrize("case", GATE, ids=[c[0] for c in GATE])
def test_prefill_parity(case):
    name, B, L, ctx, kind, ps, kv, dist = case
    w = W.make(name, 61, B, L, ctx, kind, ps, kv, dist=dist)
    log(f"[prefill] {name} ctx={w.ctx.tolist()[:4]} L={L} work-groups="
        f"{P.work_groups(B, L, w.max_seq_len, kind)}")
    host = W.build_pools_numpy(w)
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, host_pools=host)
    _untouched_rows_kept(w, d, host)


def _spread(L, n, extra):
    """n evenly spaced block tokens plus the given ones (group and block edges)."""
    return sorted({int(x) for x in np.linspace(0, L - 1, n)} | set(extra))


SCORED = [
    # name, B, L, ctx, kind, sampled block tokens
    ("pf-turn1-full-ctx80000-L753", 1, 753, 80000, W.FULL, _spread(753, 64, [0, 1, 15, 16, 751, 752])),
    ("pf-turn1-sliding-ctx80000-L753", 1, 753, 80000, W.SLIDING,
     _spread(753, 64, [0, 1, 15, 16, 751, 752])),
    ("pf-first-turn-sliding-ctx32768-L16384", 1, 16384, 32768, W.SLIDING,
     _spread(16384, 96, [0, 15, 16, 2046, 2047, 2048, 8191, 16383])),
]


@pytest.mark.parametrize("case", SCORED, ids=[c[0] for c in SCORED])
def test_prefill_full_size_sampled(case):
    name, B, L, ctx, kind, tokens = case
    w = W.make(name, 62, B, L, ctx, kind, 1, 1.0)
    log(f"[prefill] {name} pool rows={w.num_rows} checking tokens {tokens}")
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, tokens=tokens)
    assert torch.isfinite(d["out"].float()).all()
    del d
    torch.cuda.empty_cache()


def test_prefill_at_the_unit_limit():
    """4 requests x 16,384 block tokens = 4,096 plan units of 16 tokens, the
    most one call takes; the oracle recomputes sampled tokens of every request."""
    w = W.make("pf-max-units", 64, 4, 16384, (0, 100), W.FULL, 1, 1.0)
    log(f"[prefill] {w.name} ctx={w.ctx.tolist()} units={w.B * 16384 // 16}")
    d = upload(w)
    run(w, d)
    torch.cuda.synchronize()
    full_check(w, d, tokens=_spread(16384, 16, [0, 15, 16, 8191, 16383]))
    assert torch.isfinite(d["out"].float()).all()
    del d
    torch.cuda.empty_cache()


def test_prefill_partition_invariance():
    """The work-group count changes only the summation order."""
    w = W.make("pf-partition", 63, 2, 100, (1500, 2500), W.FULL, 1, 1.0)
    host = W.build_pools_numpy(w)
    d = upload(w)
    outs = []
    for g in (1, 7, 509, 0):
        log(f"[prefill partition] work_groups={g}")
        run(w, d, work_groups=g)
        outs.append(d["out"].clone())
    torch.cuda.synchronize()
    full_check(w, d, host_pools=host)
    for o in outs[:-1]:
        assert (o.float() - outs[-1].float()).abs().max().item() <= 1.6e-2
    run(w, d)
    assert torch.equal(d["out"], outs[-1]), "two identical calls differ"
