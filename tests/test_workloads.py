"""The input distributions (host only): what each draw promises holds."""
import numpy as np
import torch

from paged_fp8_kv_amd import workloads as W


def _vals(byt):
    return torch.from_numpy(byt.copy()).view(torch.float8_e4m3fn).float().numpy()


def test_soft_is_the_default_and_reproducible():
    a = W.make("s", 7, 2, 1, 500, W.FULL, 1, 1.0)
    b = W.make("s", 7, 2, 1, 500, W.FULL, 1, 1.0, dist="soft")
    for r in range(2):
        assert all(np.array_equal(x, y) for x, y in zip(a.cache_values(r), b.cache_values(r)))


def test_coherent_keys_share_a_direction():
    w = W.make("c", 8, 2, 1, 3000, W.FULL, 1, 1.0, dist="coherent")
    k, v = (_vals(x) for x in w.cache_values(1))
    for g in range(W.HKV):
        # rows against their mean direction: keys 8d + 0.1z (cos ~0.99), and on
        # full layers values 8w + 0.5z (cos ~ 8 / sqrt(64 + 16) = 0.89)
        for arr, bound in ((k[:, g], 0.98), (v[:, g], 0.85)):
            unit = arr / np.linalg.norm(arr, axis=1, keepdims=True)
            assert np.linalg.norm(unit.mean(axis=0)) > bound
    s = W.make("c", 8, 2, 1, 3000, W.SLIDING, 1, 1.0, dist="coherent")
    soft = W.make("c", 8, 2, 1, 3000, W.SLIDING, 1, 1.0)
    assert np.array_equal(s.cache_values(0)[1], soft.cache_values(0)[1])   # sliding values: soft


def test_edges_enlarge_only_the_edge_rows():
    L, ctx = 8, 6000
    soft = W.make("e", 9, 1, L, ctx, W.SLIDING, 1, 1.0)
    edge = W.make("e", 9, 1, L, ctx, W.SLIDING, 1, 1.0, dist="edges")
    ks, _ = (_vals(x) for x in soft.cache_values(0))
    ke, _ = (_vals(x) for x in edge.cache_values(0))
    differ = np.nonzero(np.any(ks != ke, axis=(1, 2)))[0]
    want = {ctx - 2048 + j for j in range(L + 1)} | {ctx - 2, ctx - 1}
    assert set(differ.tolist()) <= want and len(differ) >= len(want) - 1
    # first visible key of block token 0's window (position ctx - 2047) is enlarged
    assert np.abs(ke[ctx - 2047]).mean() > 3 * np.abs(ks[ctx - 2047]).mean()
    full = W.make("e", 9, 1, 1, ctx, W.FULL, 1, 1.0, dist="edges")
    kf, _ = (_vals(x) for x in full.cache_values(0))
    assert np.abs(kf[0]).mean() > 3 * np.abs(ks[0]).mean()


def test_outliers_enlarge_keys_only():
    soft = W.make("o", 10, 1, 1, 4000, W.FULL, 1, 1.0)
    out = W.make("o", 10, 1, 1, 4000, W.FULL, 1, 1.0, dist="outliers")
    ks, vs = (_vals(x) for x in soft.cache_values(0))
    ko, vo = (_vals(x) for x in out.cache_values(0))
    assert np.array_equal(vs, vo)
    frac = float(np.mean(ks != ko))
    assert 0.005 < frac < 0.03   # about one element in 64
    # |x| >= 6 is ~1e-9 likely for N(0,1), ~0.7% for an 8-fold draw in one element of 64
    assert np.mean(np.abs(ko) >= 6) > 0.003 and np.mean(np.abs(ks) >= 6) < 1e-4
