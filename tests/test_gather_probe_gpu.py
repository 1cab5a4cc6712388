"""museattn_gather_probe (a memory-system probe beside the step, used by the
bench for the attention kernel's ceiling) reads exactly the step's rows: the
XOR of its per-work-group checksums equals the XOR of the 32-bit words of the
K and V rows of every visible key, each once, computed on the host from the
same pools."""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
from oracle import museattn_oracle as O
from paged_fp8_kv_amd import workloads as W

from gpu_common import log, upload

pytestmark = pytest.mark.gpu


def _expected(w, kp, vp):
    acc = np.uint32(0)
    for b in range(w.B):
        n = int(w.seq_lens[b])
        u = np.arange(n)
        rows = np.array([O.cache_row(w.table, b, int(x), w.page_size) for x in u], np.int64)
        words = np.concatenate([kp[rows].reshape(len(rows), -1).view(np.uint32),
                                vp[rows].reshape(len(rows), -1).view(np.uint32)], axis=1)
        acc ^= np.bitwise_xor.reduce(words.reshape(-1))
    return int(acc)


@pytest.mark.parametrize("B,L,ctx,ps,wg", [(3, 1, (100, 5000), 1, 256), (2, 8, 9000, 64, 37),
                                           (5, 1, (1, 40), 1, 256), (2, 1, 30000, 1, 3)])
def test_gather_probe_reads_the_steps_rows(B, L, ctx, ps, wg):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = W.make(f"probe-b{B}-L{L}-p{ps}", 55, B, L, ctx, W.FULL, ps, 1.0)
    log(f"[gather probe] B={B} L={L} ctx={w.ctx.tolist()} ps={ps} work-groups={wg}")
    kp, vp = W.build_pools_numpy(w)
    d = upload(w)
    out = torch.zeros(wg, dtype=torch.int32, device="cuda")
    P.gather_probe(d["table"], d["seq_lens"], d["k_cache"], d["v_cache"], ps, w.max_seq_len, out, wg)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
    assert got == _expected(w, kp, vp)
