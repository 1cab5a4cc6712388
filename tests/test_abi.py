"""The C ABI on the host: the library loads, exports every symbol the header
declares, and its argument validation returns the documented statuses
without touching a device (fake, aligned pointer values)."""
import ctypes
import os
import re

import pytest

import paged_fp8_kv_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "museattn.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(museattn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = P.lib()
    names = _declared()
    assert set(names) == set(P.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert P.abi_version() == 1


def test_strerror_covers_all_statuses():
    for st in P.STATUS:
        assert P.strerror(st) and P.strerror(st) != "unknown status"
    assert P.strerror(12345) == "unknown status"


# fake device addresses: far apart, 256-byte aligned
BASE = 1 << 44
A = {k: BASE + i * (1 << 43) for i, k in enumerate(
    ["qkv", "pos", "table", "seq", "kc", "vc", "out", "ws", "wq", "wk", "wo"])}


def _args(**kw):
    B, L, msl, ps, kind = kw.get("B", 4), kw.get("L", 1), kw.get("max_seq_len", 1000), \
        kw.get("page_size", 1), kw.get("layer_kind", P.FULL)
    params = P.make_params(kw.get("wq", A["wq"]), A["wk"], A["wo"], kw.get("eps", 1e-6),
                           kw.get("q_scale", 5.473), kw.get("rope_base", 1e4),
                           kw.get("work_groups", 0))
    need = P.lib().museattn_workspace_bytes(B, L, msl, ps if ps in (1, 64) else 1,
                                            kind if kind in (0, 1) else 0, ctypes.byref(params))
    return dict(qkv=kw.get("qkv", A["qkv"]), positions=A["pos"], table=A["table"],
                seq_lens=A["seq"], k_cache=kw.get("kc", A["kc"]), v_cache=A["vc"],
                kv_scale=kw.get("kv_scale", 1.0), page_size=ps, layer_kind=kind,
                out=kw.get("out", A["out"]), B=B, L=L,
                table_stride=kw.get("table_stride", 1000), max_seq_len=msl,
                num_rows=kw.get("num_rows", 1 << 20), params=params,
                workspace=kw.get("ws", A["ws"]), workspace_nbytes=kw.get("ws_bytes", need))


def _check(**kw):
    return P.check_args(**_args(**kw))


def test_valid_arguments_pass():
    assert _check() == 0
    assert _check(num_rows=(1 << 32) - 1) == 0
    assert _check(page_size=64, num_rows=(1 << 32) - 64, table_stride=16) == 0
    assert _check(B=32, max_seq_len=1 << 30, table_stride=1 << 30) == 0
    assert _check(B=1024, max_seq_len=1 << 30, table_stride=1 << 30, layer_kind=P.SLIDING) == 0
    assert _check(B=1024, max_seq_len=1 << 20, table_stride=1 << 20) == 0
    assert _check(wq=A["wk"]) == 0            # read-only inputs may share memory
    assert _check(page_size=64, table_stride=16, num_rows=64 * 100) == 0
    assert _check(L=8, layer_kind=P.SLIDING) == 0
    assert _check(work_groups=65535) == 0
    assert _check(B=1024) == 0
    assert _check(L=753, max_seq_len=2000, table_stride=2000) == 0          # prefill block
    assert _check(B=4, L=16384, max_seq_len=20000, table_stride=20000) == 0  # 4 x 1024 groups


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=0), -1),
    (dict(wq=0), -1),
    (dict(ws=0), -1),
    (dict(page_size=16), -2),
    (dict(layer_kind=2), -3),
    (dict(L=16385, max_seq_len=20000), -4),
    (dict(B=300, L=753, max_seq_len=2000), -4),   # 300 x 48 token groups > 4096
    (dict(B=5, L=16384, max_seq_len=20000), -4),
    (dict(L=0), -4),
    (dict(B=0), -4),
    (dict(max_seq_len=0), -4),
    (dict(num_rows=0), -4),
    (dict(page_size=64, table_stride=100, num_rows=1000), -4),   # not a multiple of 64
    (dict(table_stride=999), -5),
    (dict(page_size=64, table_stride=15, num_rows=6400), -5),
    (dict(kc=A["kc"] + 8), -6),
    (dict(qkv=A["qkv"] + 1), -6),
    (dict(qkv=A["qkv"] + 8), -6),     # q, k, v and gate are read in 16-byte pieces
    (dict(out=A["out"] + 4), -6),     # the output is written in 8-byte pieces
    (dict(ws_bytes=1024), -7),
    (dict(ws=A["ws"] + 128), -7),
    (dict(kv_scale=0.0), -8),
    (dict(kv_scale=float("nan")), -8),
    (dict(eps=-1.0), -8),
    (dict(rope_base=0.0), -8),
    (dict(work_groups=-1), -8),
    (dict(work_groups=65536), -8),
    (dict(B=1025), -4),
    (dict(out=A["qkv"] + 4096), -9),
    (dict(out=A["kc"] + 4096), -9),          # out inside the K cache
    (dict(ws=A["vc"] + 1024), -9),           # workspace inside the V cache
    (dict(ws=A["out"]), -9),                 # workspace over out
    (dict(kc=A["vc"]), -9),                  # one array for both caches
    (dict(num_rows=1 << 32), -4),            # rows are 32-bit indices on the device
    (dict(page_size=64, num_rows=(1 << 32), table_stride=16), -4),
    # plans whose 32-bit chunk prefix sums could overflow
    (dict(B=64, max_seq_len=1 << 30, table_stride=1 << 30), -4),
    (dict(B=1024, max_seq_len=1 << 26, table_stride=1 << 26), -4),
    (dict(ws=A["pos"]), -9),                 # workspace over the positions
    (dict(out=A["table"] + 64), -9),         # out over the table
    (dict(kc=A["seq"] - 4096), -9),          # K cache over seq_lens
    (dict(ws=A["wk"] - 256), -9),            # workspace over a norm weight
])
def test_invalid_arguments_are_rejected(kw, status):
    assert _check(**kw) == status


def test_workspace_and_launch_shape():
    # one 8-wave work-group per CU of MI355X
    assert P.work_groups(32, 1, 100001, P.FULL) == 256
    assert P.work_groups(1, 8, 80008, P.SLIDING) == 256
    assert P.work_groups(1, 8, 80008, P.FULL, work_groups=7) == 7
    n = P.workspace_bytes(32, 1, 100001, 1, P.FULL)
    slots = 256 + 32
    assert n >= 34 * 4 + slots * 16 * 66 * 4
    # independent of the context length (the plan is made on the device)
    assert P.workspace_bytes(4, 8, 1 << 20, 1, P.SLIDING) == P.workspace_bytes(4, 8, 4096, 1, P.SLIDING)
    with pytest.raises(ValueError):
        P.workspace_bytes(1, 16385, 20000, 1, P.FULL)
    # prefill: partial slots per 16-token group
    n = P.workspace_bytes(1, 753, 81000, 1, P.FULL)
    units = 48
    assert n >= (units + 2) * 4 + (256 + units) * 16 * 16 * 66 * 4


def test_attn_step_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 2304, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        P.attn_step(x, torch.zeros(1, dtype=torch.int32), torch.zeros(1, 1, dtype=torch.int32),
                    torch.ones(1, dtype=torch.int32), torch.zeros(128, dtype=torch.uint8),
                    torch.zeros(128, dtype=torch.uint8), 1.0, 1, P.FULL,
                    torch.zeros(1, 1, 1024, dtype=torch.bfloat16),
                    q_norm_w=torch.ones(64), k_norm_w=torch.ones(64), o_norm_w=torch.ones(64),
                    max_seq_len=1)


@pytest.mark.parametrize("kw,status", [
    (dict(a=0), -1), (dict(o=0), -1), (dict(y=0), -1),
    (dict(T=0), -8), (dict(hidden=24), -8), (dict(hidden=0), -8), (dict(hidden=65552), -8),
    (dict(a=A["qkv"] + 8), -6), (dict(o=A["wq"] + 4), -6), (dict(y=A["out"] + 4), -6),
    (dict(y=A["qkv"]), -9),
])
def test_oproj_invalid_arguments_are_rejected(kw, status):
    """Host-side checks of museattn_oproj: they return before any device call."""
    lib = P.lib()
    args = dict(a=A["qkv"], o=A["wq"], T=4, hidden=8192, y=A["out"])
    args.update(kw)
    st = lib.museattn_oproj(args["a"], args["o"], args["T"], args["hidden"], args["y"], None)
    assert st == status


@pytest.mark.parametrize("y_at,status", [("ws", -9), ("kc", -9), ("qkv", -9), ("wk", 0)])
def test_step_oproj_output_must_not_overlap(y_at, status):
    """museattn_attn_step_oproj: y may not overlap qkv, the caches or the
    workspace (host checks only; an invalid call enqueues nothing, and the
    valid one is not run: the check order is probed with a null o_weight)."""
    lib = P.lib()
    kw = _args()
    o_w = 0 if status == 0 else A["wq"] + (1 << 30)
    st = lib.museattn_attn_step_oproj(
        kw["qkv"], kw["positions"], kw["table"], kw["seq_lens"], kw["k_cache"], kw["v_cache"],
        kw["kv_scale"], kw["page_size"], kw["layer_kind"], kw["out"], None, kw["B"], kw["L"],
        kw["table_stride"], kw["max_seq_len"], kw["num_rows"], ctypes.byref(kw["params"]),
        kw["workspace"], kw["workspace_nbytes"], o_w, 8192, A[y_at] + 4096, None, None)
    assert st == (status if status else -1)


@pytest.mark.parametrize("kw,status", [
    (dict(table=0), -1), (dict(out=0), -1), (dict(ps=16), -2), (dict(B=0), -4),
    (dict(B=1025), -4), (dict(msl=0), -4), (dict(rows=1 << 32), -4), (dict(stride=999), -5),
    (dict(wg=0), -8), (dict(wg=65536), -8), (dict(kc=A["kc"] + 8), -6), (dict(out=A["ws"] + 2), -6),
])
def test_gather_probe_invalid_arguments_are_rejected(kw, status):
    """Host-side checks of museattn_gather_probe: they return before any device call."""
    a = dict(table=A["table"], seq=A["seq"], kc=A["kc"], vc=A["vc"], ps=1, B=4, stride=1000,
             msl=1000, rows=1 << 20, out=A["ws"], wg=256)
    a.update(kw)
    st = P.lib().museattn_gather_probe(a["table"], a["seq"], a["kc"], a["vc"], a["ps"], a["B"],
                                       a["stride"], a["msl"], a["rows"], a["out"], a["wg"], None)
    assert st == status
