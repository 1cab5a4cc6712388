"""Pins for the CPU oracle: what the format, the mathematics and library
routines fix, independently of the oracle's own code (CPU only).

The pages print no worked numbers for this step, so the oracle is pinned by
the FP8 format definition, closed forms, invariants, and an independent
re-statement of the whole step on PyTorch library routines (rms_norm,
complex multiplication, scaled_dot_product_attention with an explicit mask).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import museattn_oracle as O
from paged_fp8_kv_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = float(np.float32(1e-6))
QS = float(np.float32(5.473))


# ----------------------------------------------------------------- FP8 codec

def _golden_codes():
    out = []
    with open(os.path.join(GOLDEN, "e4m3fn_spec_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                out.append((int(c, 16), float(v)))
    return out


def test_e4m3_decode_spec_values():
    for c, v in _golden_codes():
        got = O.e4m3_decode(c)
        if math.isnan(v):
            assert np.isnan(got), hex(c)
        else:
            assert got == v and bool(np.signbit(got)) == (math.copysign(1, v) < 0), (hex(c), got, v)


def test_e4m3_decode_matches_library_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_decode(np.arange(256))
    same = (lib == ours) | (np.isnan(lib) & np.isnan(ours))
    assert same.all()


def test_e4m3_encode_matches_library_cast_on_all_bf16():
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    x = bits[np.isfinite(bits) & (np.abs(bits) < 448)]
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = O.e4m3_encode(x)
    assert (lib == ours).all()


def test_e4m3_roundtrip_and_order():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert (O.e4m3_encode(O.e4m3_decode(codes)) == codes).all()
    v = O.e4m3_decode(np.arange(127))
    assert (np.diff(v) > 0).all()


def test_e4m3_ties_to_even_and_neighbours():
    v = O.e4m3_decode(np.arange(127))
    mids = 0.5 * (v[:-1] + v[1:])
    got = O.e4m3_encode(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert (got == want).all()
    assert (O.e4m3_encode(np.nextafter(mids, 0)) == lo).all()
    assert (O.e4m3_encode(np.nextafter(mids, 1e9)) == lo + 1).all()


def test_e4m3_saturates_at_448():
    big = np.array([448.0, 448.0001, 460.0, 464.0, 500.0, 1e6, np.inf])
    assert (O.e4m3_encode(big) == 0x7E).all()
    assert (O.e4m3_encode(-big) == 0xFE).all()
    assert O.e4m3_encode(2.0 ** -10) == 0x00          # tie between 0 and 2^-9 -> even
    assert O.e4m3_encode(-1e-6) == 0x80                # sign kept on underflow
    assert O.e4m3_encode(1.5 * 2.0 ** -10) == 0x01


def test_e4m3_ordinal():
    assert O.e4m3_ordinal(0x00) == O.e4m3_ordinal(0x80) == 0
    assert O.e4m3_ordinal(0x01) - O.e4m3_ordinal(0x81) == 2
    assert O.e4m3_ordinal(0x7E) == 126 and O.e4m3_ordinal(0xFE) == -126


# ------------------------------------------------------------- rmsnorm, RoPE

def test_rmsnorm_matches_library_and_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    w = 1 + 0.1 * rng.standard_normal(64)
    lib = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), 1e-6).numpy()
    assert np.allclose(O.rmsnorm(x, w, 1e-6), lib, rtol=1e-13, atol=1e-13)
    c = np.full(64, -3.0)
    assert np.allclose(O.rmsnorm(c, w, 0.0), -w, rtol=1e-15)
    assert np.allclose(O.rmsnorm(7.5 * x, w, 0.0), O.rmsnorm(x, w, 0.0), rtol=1e-13)


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(64)
    assert np.array_equal(O.rope_neox(x, 0, 10000.0), x)
    for p in (1, 17, 2047, 80000, 1048575):
        y = O.rope_neox(x, p, 10000.0)
        assert np.allclose(x[:32] ** 2 + x[32:] ** 2, y[:32] ** 2 + y[32:] ** 2, rtol=1e-12)


def test_rope_first_pair_is_a_complex_rotation_by_p_radians():
    # inv_0 = base^0 = 1 exactly, so pair (0, 32) turns by exactly p radians.
    rng = np.random.default_rng(3)
    x = rng.standard_normal(64)
    for p in (1, 3, 1000, 80000):
        y = O.rope_neox(x, p, 10000.0)
        z = complex(x[0], x[32]) * complex(math.cos(p), math.sin(p))
        assert abs(y[0] - z.real) < 1e-12 and abs(y[32] - z.imag) < 1e-12


def test_rope_inverse_frequencies():
    inv = O.rope_inv_freq(10000.0)
    alt = np.array([math.exp(-i / 32 * math.log(10000.0)) for i in range(32)], dtype=np.float32)
    ulp = np.spacing(alt.astype(np.float32)).astype(np.float64)
    assert (np.abs(inv - alt.astype(np.float64)) <= ulp).all()
    assert inv[0] == 1.0 and inv[16] == np.float32(0.01)


def test_rope_relative_position_property():
    # <R_p q, R_p' k> depends only on p - p' when every angle is exact in fp32
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    d1 = O.rope_neox(q, 40, 10000.0) @ O.rope_neox(k, 30, 10000.0)
    d2 = O.rope_neox(q, 12, 10000.0) @ O.rope_neox(k, 2, 10000.0)
    assert abs(d1 - d2) < 1e-5 * (np.abs(q).sum() * np.abs(k).sum())


# -------------------------------------------- whole step vs library routines

def _tiny(B, L, ctx, kind, ps, kv=1.0, seed=7, pool_rows=None):
    return W.make("tiny", seed, B, L, ctx, kind, ps, kv, pool_rows)


def _run_oracle(w, kp, vp, **kw):
    return O.attn_step(w.qkv.float().numpy(), w.positions, w.table, kp, vp, B=w.B, L=w.L,
                       page_size=w.page_size, layer_kind=w.layer_kind, kv_scale=w.kv_scale,
                       w_q=w.w_q, w_k=w.w_k, w_o=w.w_o, eps=EPS, q_scale=QS, **kw)


def _rope_complex(x, pos):
    """Rotation written as complex multiplication (torch.polar), fp32 angles."""
    inv = torch.tensor([np.float32(10000.0 ** (-i / 32)) for i in range(32)], dtype=torch.float32)
    th = (pos.to(torch.float32)[:, None] * inv[None, :]).to(torch.float64)   # [T, 32]
    z = torch.complex(x[..., :32], x[..., 32:]) * torch.polar(torch.ones_like(th), th)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def _library_step(w, kp, vp):
    """The page's listing on PyTorch library routines (independent of the oracle)."""
    T = w.T
    x = w.qkv.to(torch.float64)
    q = x[:, :1024].reshape(T, 16, 64)
    k = x[:, 1024:1152].reshape(T, 2, 64)
    v = x[:, 1152:1280].reshape(T, 2, 64)
    g = x[:, 1280:].reshape(T, 16, 64)
    q = F.rms_norm(q, (64,), torch.from_numpy(w.w_q).double(), EPS) * QS
    k = F.rms_norm(k, (64,), torch.from_numpy(w.w_k).double(), EPS)
    pos = torch.from_numpy(w.positions.astype(np.int64))
    sliding = w.layer_kind == W.SLIDING
    if sliding:
        q, k = _rope_complex(q, pos), _rope_complex(k, pos)
    kv = w.kv_scale
    kb = (k / kv).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vb = (v / kv).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kp, vp = kp.copy(), vp.copy()
    ps = w.page_size
    for t in range(T):
        b, p = t // w.L, int(w.positions[t])
        r = int(w.table[b, p // ps]) * ps + p % ps
        kp[r], vp[r] = kb[t], vb[t]
    out = torch.zeros(T, 16, 64, dtype=torch.float64)
    for b in range(w.B):
        n = int(w.seq_lens[b])
        u = np.arange(n)
        rows = w.table[b, u // ps].astype(np.int64) * ps + u % ps
        K = torch.from_numpy(kp[rows]).view(torch.float8_e4m3fn).to(torch.float64) * kv
        V = torch.from_numpy(vp[rows]).view(torch.float8_e4m3fn).to(torch.float64) * kv
        Q = q[b * w.L:(b + 1) * w.L].permute(1, 0, 2)[None]           # [1, 16, L, 64]
        pj = pos[b * w.L:(b + 1) * w.L][:, None]
        uu = torch.arange(n)[None, :]
        mask = uu <= pj
        if sliding:
            mask &= uu >= pj - 2047
        a = F.scaled_dot_product_attention(Q, K.permute(1, 0, 2)[None], V.permute(1, 0, 2)[None],
                                           attn_mask=mask, enable_gqa=True)
        out[b * w.L:(b + 1) * w.L] = a[0].permute(1, 0, 2)
    res = F.rms_norm(out, (64,), torch.from_numpy(w.w_o).double(), EPS) * torch.sigmoid(g)
    return res.reshape(w.B, w.L, 1024).numpy(), kb, vb


CASES = [
    # B, L, ctx, kind, page_size, kv_scale
    (1, 1, 0, W.FULL, 1, 1.0),
    (1, 1, 40, W.FULL, 1, 1.0),
    (2, 1, (10, 90), W.SLIDING, 1, 1.0),
    (1, 8, 33, W.FULL, 1, 1.0),
    (2, 8, 70, W.SLIDING, 64, 1.0),
    (3, 8, (2040, 2060), W.SLIDING, 1, 1.0),     # window edges inside the block
    (2, 1, (2100, 2300), W.SLIDING, 64, 1.0 / 64),
    (2, 4, (100, 300), W.FULL, 64, 1.0 / 64),
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_library_restatement(case):
    B, L, ctx, kind, ps, kv = case
    w = _tiny(B, L, ctx, kind, ps, kv)
    kp, vp = W.build_pools_numpy(w)
    want, kb, vb = _library_step(w, kp, vp)
    got, okb, ovb = _run_oracle(w, kp.copy(), vp.copy())
    assert (okb == kb).all() and (ovb == vb).all()
    assert np.abs(got - want).max() < 1e-9


def _max_err_vs_library(case):
    B, L, ctx, kind, ps, kv = case
    w = _tiny(B, L, ctx, kind, ps, kv)
    kp, vp = W.build_pools_numpy(w)
    want, _, _ = _library_step(w, kp, vp)
    try:
        got, _, _ = _run_oracle(w, kp.copy(), vp.copy())
    except Exception:
        return math.inf
    err = float(np.abs(got - want).max())
    return err if math.isfinite(err) else math.inf   # NaN (sentinel rows read) is an error


def _with_kw(fn, **over):
    """fn with some keyword arguments forced (a planted mistake)."""
    return lambda *a, **k: fn(*a, **{**k, **over})


def _with_args(fn, over):
    """fn with some positional arguments forced (a planted mistake)."""
    def g(*a, **k):
        a = list(a)
        for i, v in over.items():
            a[i] = v
        return fn(*a, **k)
    return g


def _rope_interleaved(x, p, base):
    """The other common RoPE layout, pairs (2i, 2i + 1): a plausible mix-up."""
    x = np.asarray(x, dtype=np.float64)
    th = O.rope_angles(p, base)
    c, s = np.cos(th), np.sin(th)
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2], y[..., 1::2] = a * c - b * s, b * c + a * s
    return y


MUTANTS = {
    "softmax divisor 4": lambda mp: mp.setattr(O, "SOFTMAX_DIV", 4.0),
    "groups of 4 heads": lambda mp: mp.setattr(O, "GROUP", 4),
    "window one short": lambda mp: mp.setattr(O, "visible_keys",
                                              lambda p, w: (0 if w is None else max(0, p - (w - 2)), p)),
    "no causal mask": lambda mp: mp.setattr(O, "visible_keys",
                                            lambda p, w: (0 if w is None else max(0, p - (w - 1)), p + 1)),
    "rope sign": lambda mp: mp.setattr(O, "rope_angles", lambda p, base: -O.rope_inv_freq(base) * p),
    "gate not applied": lambda mp: mp.setattr(O, "sigmoid", lambda x: np.ones_like(x)),
    "q scale dropped": lambda mp: mp.setattr(
        O, "prologue", _with_kw(O.prologue, q_scale=1.0)),
    "rope on full layers too": lambda mp: mp.setattr(
        O, "prologue", _with_kw(O.prologue, rope=True)),
    "kv_scale not applied on read": lambda mp: mp.setattr(
        O, "attend", _with_args(O.attend, {8: 1.0})),
    "rmsnorm sums instead of means": lambda mp: mp.setattr(
        O, "rmsnorm", lambda x, w, eps: np.asarray(x, np.float64) / np.sqrt(
            np.sum(np.asarray(x, np.float64) ** 2, axis=-1, keepdims=True) + eps) * w),
    "output norm weight ignored": lambda mp: mp.setattr(
        O, "gated_output", lambda a, gate, w_o, eps: O.rmsnorm(a, np.ones_like(w_o), eps)
        * O.sigmoid(gate)),
    "rope pairs adjacent dims": lambda mp: mp.setattr(O, "rope_neox", _rope_interleaved),
    "k and v slices swapped": lambda mp: (mp.setattr(O, "K_OFF", O.V_OFF),
                                          mp.setattr(O, "V_OFF", O.K_OFF)),
    "page offset dropped": lambda mp: mp.setattr(
        O, "cache_row", lambda table, b, u, ps: table[b, np.asarray(u, np.int64) // ps]
        .astype(np.int64) * ps),
    "new rows not written": lambda mp: mp.setattr(O, "write_rows", lambda *a, **k: None),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_oracle_mistakes_are_caught(monkeypatch, name):
    # each plausible mistake, planted in the oracle, must break the library pin
    cases = [(3, 8, (2040, 2060), W.SLIDING, 1, 1.0), (2, 4, (100, 300), W.FULL, 64, 1.0 / 64)]
    MUTANTS[name](monkeypatch)
    worst = max(_max_err_vs_library(c) for c in cases)
    assert worst > 1e-3, name


# ---------------------------------------------------------------- invariants

def test_empty_context_returns_new_value():
    w = _tiny(2, 1, 0, W.FULL, 1)
    kp, vp = W.build_pools_numpy(w)
    out, _, vb = _run_oracle(w, kp, vp)
    a = np.repeat(O.e4m3_decode(vb), 8, axis=1)             # head h reads KV head h // 8
    gate = w.qkv.float().numpy()[:, 1280:].reshape(2, 16, 64)
    want = O.rmsnorm(a, w.w_o, EPS) * O.sigmoid(gate)
    assert np.allclose(out.reshape(2, 16, 64), want, rtol=1e-13, atol=1e-13)


def test_constant_value_rows_give_closed_form():
    w = _tiny(2, 8, 300, W.SLIDING, 1)
    rng = np.random.default_rng(5)
    codes = rng.integers(0x08, 0x70, size=(2, 64)).astype(np.uint8)   # normal, moderate values
    codes[:, ::3] |= 0x80
    kp, vp = W.build_pools_numpy(w)
    vp[:] = codes[None]
    vals = O.e4m3_decode(codes)                          # exactly representable in bf16
    qkv = w.qkv.clone()
    qkv[:, 1152:1280] = torch.from_numpy(vals.reshape(-1)).to(torch.bfloat16)[None]
    w.qkv = qkv
    out, _, vb = _run_oracle(w, kp, vp)
    assert (vb == codes[None]).all()
    gate = qkv.float().numpy()[:, 1280:].reshape(-1, 16, 64)
    want = O.rmsnorm(np.repeat(vals[None], 8, axis=1), w.w_o, EPS) * O.sigmoid(gate)
    assert np.allclose(out.reshape(-1, 16, 64), want, rtol=1e-12, atol=1e-12)


def test_window_equals_full_when_context_fits():
    w = _tiny(2, 8, (1000, 2040), W.SLIDING, 1)     # ctx + L <= 2048
    kp, vp = W.build_pools_numpy(w)
    x = w.qkv.float().numpy()
    q, kb, vb, gate = O.prologue(x, w.positions, w.w_q, w.w_k, eps=EPS, q_scale=QS, rope=True,
                                 rope_base=10000.0, kv_scale=1.0)
    O.write_rows(kp, vp, w.table, w.positions, w.B, w.L, 1, kb, vb)
    a_win = O.attend(q, kp, vp, w.table, w.positions, w.B, w.L, 1, 1.0, 2048)
    a_full = O.attend(q, kp, vp, w.table, w.positions, w.B, w.L, 1, 1.0, None)
    assert np.array_equal(a_win, a_full)


def test_page_layout_and_row_permutation_do_not_matter():
    # same seed and contexts -> same logical cache; the pool size and page size
    # change only where the rows land
    outs = []
    for ps, pool in ((1, None), (1, 5003), (64, None), (64, 64 * 40)):
        w = W.make("perm", 11, 2, 8, (150, 200), W.FULL, ps, 1.0, pool)
        kp, vp = W.build_pools_numpy(w)
        outs.append(_run_oracle(w, kp, vp)[0])
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


def test_kv_scale_power_of_two_is_exact():
    # bytes fp8(64 x) read at kv_scale 1/64 equal bytes fp8(x) at kv_scale 1
    # wherever both are normal and unsaturated (|x| in [2^-6, 7])
    wa = _tiny(1, 8, 500, W.FULL, 1, kv=1.0, seed=13)
    wb = _tiny(1, 8, 500, W.FULL, 1, kv=1.0 / 64, seed=13)
    ka, va = W.build_pools_numpy(wa)

    def in_range(c):
        d = np.abs(O.e4m3_decode(c))
        return (d >= 2 ** -6) & (d <= 7)

    ka = np.where(in_range(ka), ka, 0x38).astype(np.uint8)
    va = np.where(in_range(va), va, 0xB8).astype(np.uint8)
    kb = O.e4m3_encode(O.e4m3_decode(ka) * 64)
    vb = O.e4m3_encode(O.e4m3_decode(va) * 64)
    assert (O.e4m3_ordinal(kb) - O.e4m3_ordinal(ka) == np.where(ka & 0x80, -48, 48)).all()
    # new tokens: k = +-1 per dim (rmsnorm gives +-w_k), v = +-0.5
    qkv = wa.qkv.clone()
    x = qkv[:, 1024:1280].float()
    qkv[:, 1024:1152] = torch.where(x[:, :128] < 0, -1.0, 1.0).to(torch.bfloat16)
    qkv[:, 1152:1280] = torch.where(x[:, 128:] < 0, -0.5, 0.5).to(torch.bfloat16)
    wa.qkv, wb.qkv = qkv, qkv.clone()
    oa, kba, vba = _run_oracle(wa, ka, va)
    ob, kbb, vbb = _run_oracle(wb, kb, vb)
    assert in_range(kba).all() and in_range(vba).all()
    assert (O.e4m3_ordinal(kbb) - O.e4m3_ordinal(kba) == np.where(kba & 0x80, -48, 48)).all()
    assert np.array_equal(oa, ob)


def test_causality_inside_the_block():
    w = _tiny(1, 8, 60, W.FULL, 1, seed=17)
    kp, vp = W.build_pools_numpy(w)
    o1, _, _ = _run_oracle(w, kp.copy(), vp.copy())
    qkv = w.qkv.clone()
    qkv[5:] = torch.randn(3, 2304, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    w.qkv = qkv
    o2, _, _ = _run_oracle(w, kp.copy(), vp.copy())
    assert np.array_equal(o1[0, :5], o2[0, :5])
    assert not np.array_equal(o1[0, 5:], o2[0, 5:])


def test_requests_are_independent():
    w = _tiny(3, 2, (50, 80), W.FULL, 1, seed=19)
    kp, vp = W.build_pools_numpy(w)
    o1, _, _ = _run_oracle(w, kp.copy(), vp.copy())
    qkv = w.qkv.clone()
    qkv[0:2] = 0.5
    w.qkv = qkv
    o2, _, _ = _run_oracle(w, kp.copy(), vp.copy())
    assert np.array_equal(o1[1:], o2[1:]) and not np.array_equal(o1[0], o2[0])


# --------------------------------------------------------------------------
# The output projection (task page "Whole decoder layer", section "What to
# compute": y = out @ o^T): pinned by closed forms and brute force, not by the
# matmul it calls.
# --------------------------------------------------------------------------

def test_oproj_permutation_rows_select_inputs():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((5, 1024))
    perm = rng.permutation(1024)[:48]
    o = np.zeros((48, 1024))
    o[np.arange(48), perm] = 1.0          # row n picks input feature perm[n]
    y = O.oproj(a, o)
    assert np.array_equal(y, a[:, perm])
    o2 = o * 3.0                           # linear in o
    assert np.array_equal(O.oproj(a, o2), 3.0 * a[:, perm])


def test_oproj_brute_force_on_small_inputs():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((3, 1024))
    o = rng.standard_normal((16, 1024))
    y = O.oproj(a, o)
    for t in range(3):
        for n in range(16):
            want = math.fsum(float(a[t, k]) * float(o[n, k]) for k in range(1024))
            assert abs(y[t, n] - want) <= 1e-9 * (1 + abs(want))


def test_oproj_catches_a_transposed_operand(monkeypatch):
    # a square, non-symmetric o: using o instead of o^T must be seen
    rng = np.random.default_rng(9)
    a = rng.standard_normal((4, 1024))
    o = rng.standard_normal((1024, 1024))
    brute = np.array([[math.fsum(a[t] * o[n]) for n in range(0, 1024, 97)] for t in range(4)])
    assert np.allclose(O.oproj(a, o)[:, ::97], brute, rtol=1e-9, atol=1e-9)
    monkeypatch.setattr(O, "oproj", lambda a_, o_: np.asarray(a_) @ np.asarray(o_))
    assert not np.allclose(O.oproj(a, o)[:, ::97], brute, rtol=1e-3, atol=1e-3)
