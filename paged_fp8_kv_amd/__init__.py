"""Python binding of libmuseattn (argument marshalling only).

Every step of the attention computation runs in the library's HIP kernels;
this module checks tensor dtypes, shapes, devices and contiguity, and passes
raw device pointers and the current HIP stream to the C ABI declared in
include/museattn.h.  There is no fallback: if the library is not built, the
calls raise.

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# MUSEATTN_LIB may name another build of the library (the instrumented
# libmuseattn_phases.so that bench.py --phases loads)
LIB_PATH = os.environ.get("MUSEATTN_LIB") or os.path.join(HERE, "libmuseattn.so")

FULL, SLIDING = 0, 1
HQ, HKV, D = 16, 2, 64
QKV_WIDTH, OUT_WIDTH, ROW_BYTES = 2304, 1024, 128
DEFAULT_EPS, DEFAULT_Q_SCALE, DEFAULT_ROPE_BASE = 1e-6, 5.473, 10000.0

OK = 0
STATUS = {
    0: "MUSEATTN_OK", -1: "MUSEATTN_ERR_NULL", -2: "MUSEATTN_ERR_PAGE_SIZE",
    -3: "MUSEATTN_ERR_LAYER_KIND", -4: "MUSEATTN_ERR_SHAPE", -5: "MUSEATTN_ERR_TABLE",
    -6: "MUSEATTN_ERR_ALIGN", -7: "MUSEATTN_ERR_WORKSPACE", -8: "MUSEATTN_ERR_PARAM",
    -9: "MUSEATTN_ERR_ALIAS", -10: "MUSEATTN_ERR_LAUNCH",
}

# every symbol include/museattn.h declares
EXPORTS = ("museattn_abi_version", "museattn_strerror", "museattn_workspace_bytes",
           "museattn_check_args", "museattn_attn_step", "museattn_attn_step_profiled",
           "museattn_work_groups", "museattn_oproj", "museattn_attn_step_oproj",
           "museattn_attn_step_noalloc", "museattn_gather_probe")
STATIC_SCRATCH_BYTES = 32 << 20   # MUSEATTN_STATIC_SCRATCH_BYTES


class Params(ctypes.Structure):
    _fields_ = [
        ("q_norm_w", ctypes.c_void_p),
        ("k_norm_w", ctypes.c_void_p),
        ("o_norm_w", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("q_scale", ctypes.c_float),
        ("rope_base", ctypes.c_float),
        ("work_groups", ctypes.c_int),
    ]


class MuseAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({strerror(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmuseattn is not built ({LIB_PATH} missing); run "
                               "`python -m paged_fp8_kv_amd.build` or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        pp = ctypes.POINTER(Params)
        L.museattn_abi_version.restype = i32
        L.museattn_abi_version.argtypes = []
        L.museattn_strerror.restype = ctypes.c_char_p
        L.museattn_strerror.argtypes = [i32]
        L.museattn_workspace_bytes.restype = ctypes.c_size_t
        L.museattn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, pp]
        L.museattn_work_groups.restype = i32
        L.museattn_work_groups.argtypes = [i32, i32, i32, i32, pp]
        common = [vp, vp, vp, vp, vp, vp, f32, i32, i32, vp]
        L.museattn_check_args.restype = i32
        L.museattn_check_args.argtypes = common + [i32, i32, i32, i32, i64, pp, vp, ctypes.c_size_t]
        L.museattn_attn_step.restype = i32
        L.museattn_attn_step.argtypes = common + [vp, i32, i32, i32, i32, i64, pp, vp,
                                                  ctypes.c_size_t]
        L.museattn_attn_step_profiled.restype = i32
        L.museattn_attn_step_profiled.argtypes = L.museattn_attn_step.argtypes + [vp, vp]
        L.museattn_attn_step_oproj.restype = i32
        L.museattn_attn_step_oproj.argtypes = L.museattn_attn_step.argtypes + [vp, i32, vp, vp, vp]
        L.museattn_attn_step_noalloc.restype = i32
        L.museattn_attn_step_noalloc.argtypes = common + [vp, i32, i32, i32, i32, i64, pp]
        L.museattn_gather_probe.restype = i32
        L.museattn_gather_probe.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i64, vp, i32, vp]
        L.museattn_oproj.restype = i32
        L.museattn_oproj.argtypes = [vp, vp, i32, i32, vp, vp]
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().museattn_abi_version()


def strerror(status: int) -> str:
    return lib().museattn_strerror(int(status)).decode()


def make_params(q_norm_w=0, k_norm_w=0, o_norm_w=0, eps=DEFAULT_EPS, q_scale=DEFAULT_Q_SCALE,
                rope_base=DEFAULT_ROPE_BASE, work_groups=0) -> Params:
    """Params from device pointers (ints) or tensors."""
    ptr = lambda x: x.data_ptr() if hasattr(x, "data_ptr") else int(x)  # noqa: E731
    return Params(ptr(q_norm_w), ptr(k_norm_w), ptr(o_norm_w), float(eps), float(q_scale),
                  float(rope_base), int(work_groups))


def workspace_bytes(B, L, max_seq_len, page_size, layer_kind, work_groups=0) -> int:
    p = make_params(work_groups=work_groups)
    n = lib().museattn_workspace_bytes(int(B), int(L), int(max_seq_len), int(page_size),
                                       int(layer_kind), ctypes.byref(p))
    if n == 0:
        raise ValueError("museattn_workspace_bytes: invalid shapes")
    return n


def work_groups(B, L, max_seq_len, layer_kind, work_groups=0) -> int:
    p = make_params(work_groups=work_groups)
    return lib().museattn_work_groups(int(B), int(L), int(max_seq_len), int(layer_kind),
                                      ctypes.byref(p))


def check_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
               layer_kind, out, B, L, table_stride, max_seq_len, num_rows, params,
               workspace, workspace_nbytes) -> int:
    """museattn_check_args on raw pointers (ints); host only."""
    return lib().museattn_check_args(qkv, positions, table, seq_lens, k_cache, v_cache,
                                     float(kv_scale), int(page_size), int(layer_kind), out,
                                     int(B), int(L), int(table_stride), int(max_seq_len),
                                     int(num_rows), ctypes.byref(params), workspace,
                                     int(workspace_nbytes))


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _step_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
               layer_kind, out, stream, q_norm_w, k_norm_w, o_norm_w, max_seq_len, eps,
               q_scale, rope_base, work_groups):
    """Checks the step's tensors; returns the C arguments up to `params`,
    the params struct (kept alive by the caller) and B, L."""
    import torch

    B = int(seq_lens.shape[0])
    _need(out.dim() == 3 and out.shape[0] == B and out.shape[2] == OUT_WIDTH, "out must be [B, L, 1024]")
    L = int(out.shape[1])
    T = B * L
    tensors = dict(qkv=qkv, positions=positions, table=table, seq_lens=seq_lens, k_cache=k_cache,
                   v_cache=v_cache, out=out, q_norm_w=q_norm_w, k_norm_w=k_norm_w,
                   o_norm_w=o_norm_w)
    dev = qkv.device
    for name, t in tensors.items():
        _need(t.is_cuda and t.device == dev, f"{name} must be on {dev}")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(qkv.dtype == torch.bfloat16 and tuple(qkv.shape) == (T, QKV_WIDTH), "qkv must be bf16 [B*L, 2304]")
    _need(out.dtype == torch.bfloat16, "out must be bf16")
    _need(positions.dtype == torch.int32 and positions.numel() == T, "positions must be int32 [B*L]")
    _need(seq_lens.dtype == torch.int32, "seq_lens must be int32 [B]")
    _need(table.dtype == torch.int32 and table.dim() == 2 and table.shape[0] == B, "table must be int32 [B, stride]")
    for name in ("q_norm_w", "k_norm_w", "o_norm_w"):
        t = tensors[name]
        _need(t.dtype == torch.float32 and t.numel() == D, f"{name} must be float32 [64]")
    for name in ("k_cache", "v_cache"):
        t = tensors[name]
        _need(t.dtype == torch.uint8 and t.numel() % ROW_BYTES == 0, f"{name} must be uint8 rows of 128 B")
    _need(k_cache.numel() == v_cache.numel(), "k_cache and v_cache must hold the same rows")
    num_rows = k_cache.numel() // ROW_BYTES
    params = make_params(q_norm_w, k_norm_w, o_norm_w, eps, q_scale, rope_base, work_groups)
    if stream is None:
        stream_ptr = torch.cuda.current_stream(dev).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream_ptr = stream.cuda_stream
    else:
        stream_ptr = int(stream)
    args = (qkv.data_ptr(), positions.data_ptr(), table.data_ptr(), seq_lens.data_ptr(),
            k_cache.data_ptr(), v_cache.data_ptr(), float(kv_scale), int(page_size),
            int(layer_kind), out.data_ptr(), stream_ptr, B, L, int(table.shape[1]),
            int(max_seq_len), int(num_rows), ctypes.byref(params))
    return args, params, B, L


def attn_step(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
              layer_kind, out, stream=None, *, q_norm_w, k_norm_w, o_norm_w, max_seq_len,
              workspace=None, eps=DEFAULT_EPS, q_scale=DEFAULT_Q_SCALE,
              rope_base=DEFAULT_ROPE_BASE, work_groups=0, attn_events=None, o_weight=None,
              y=None, oproj_events=None):
    """One attention step on torch tensors (see include/museattn.h).

    qkv bf16 [B*L, 2304]; positions int32 [B*L]; table int32 [B, stride];
    seq_lens int32 [B]; k_cache / v_cache uint8 [num_rows, 2, 64] (or any
    uint8 view of that many bytes); out bf16 [B, L, 1024]; norm weights
    float32 [64]; workspace uint8 of >= workspace_bytes(...) bytes or None
    (then allocated here with torch).  stream: a torch.cuda.Stream, a raw
    hipStream_t int, or None for the current stream.  attn_events: optional
    (start, end) torch.cuda.Event pair recorded around the attention kernel
    (museattn_attn_step_profiled).  o_weight (bf16 [hidden, 1024]) and y
    (bf16 [B*L, hidden]) given: the output projection follows the step
    (museattn_attn_step_oproj), oproj_events around its kernel."""
    import torch

    args, params, B, L = _step_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale,
                                     page_size, layer_kind, out, stream, q_norm_w, k_norm_w,
                                     o_norm_w, max_seq_len, eps, q_scale, rope_base, work_groups)
    T = B * L
    dev = qkv.device
    need = workspace_bytes(B, L, max_seq_len, page_size, layer_kind, work_groups)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace.is_cuda and workspace.device == dev and workspace.dtype == torch.uint8
          and workspace.is_contiguous(),
          f"workspace must be a contiguous uint8 tensor on {dev}")   # one span of numel bytes
    args = args + (workspace.data_ptr(), int(workspace.numel()))
    if o_weight is not None or y is not None:
        _need(o_weight is not None and y is not None, "o_weight and y go together")
        _need(attn_events is None, "attn_events are not recorded with the projection")
        hidden = _check_oproj(out.view(T, OUT_WIDTH), o_weight, y, dev)
        ev = oproj_events or (None, None)
        st = lib().museattn_attn_step_oproj(*args, o_weight.data_ptr(), hidden, y.data_ptr(),
                                            ev[0].cuda_event if ev[0] is not None else None,
                                            ev[1].cuda_event if ev[1] is not None else None)
        if st != OK:
            raise MuseAttnError(st, "museattn_attn_step_oproj")
        return out
    if attn_events is None:
        st = lib().museattn_attn_step(*args)
    else:
        st = lib().museattn_attn_step_profiled(*args, attn_events[0].cuda_event,
                                               attn_events[1].cuda_event)
    if st != OK:
        raise MuseAttnError(st, "museattn_attn_step")
    return out


def attn_step_noalloc(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale, page_size,
                      layer_kind, out, stream=None, *, q_norm_w, k_norm_w, o_norm_w,
                      max_seq_len, eps=DEFAULT_EPS, q_scale=DEFAULT_Q_SCALE,
                      rope_base=DEFAULT_ROPE_BASE, work_groups=0):
    """museattn_attn_step_noalloc: the step with its scratch in the library's
    static device array (no allocation by the library or here).  Calls that may
    overlap on one GPU race on that array."""
    args, params, B, L = _step_args(qkv, positions, table, seq_lens, k_cache, v_cache, kv_scale,
                                     page_size, layer_kind, out, stream, q_norm_w, k_norm_w,
                                     o_norm_w, max_seq_len, eps, q_scale, rope_base, work_groups)
    st = lib().museattn_attn_step_noalloc(*args)
    if st != OK:
        raise MuseAttnError(st, "museattn_attn_step_noalloc")
    return out


def _check_oproj(a, o_weight, y, dev) -> int:
    import torch
    for name, t in (("a", a), ("o_weight", o_weight), ("y", y)):
        _need(t.is_cuda and t.device == dev, f"{name} must be on {dev}")
        _need(t.is_contiguous() and t.dtype == torch.bfloat16, f"{name} must be contiguous bf16")
    _need(o_weight.dim() == 2 and o_weight.shape[1] == OUT_WIDTH, "o_weight must be [hidden, 1024]")
    hidden = int(o_weight.shape[0])
    _need(a.dim() == 2 and a.shape[1] == OUT_WIDTH, "a must be [T, 1024]")
    _need(tuple(y.shape) == (a.shape[0], hidden), "y must be [T, hidden]")
    return hidden


def oproj(a, o_weight, y, stream=None):
    """museattn_oproj: y = a @ o_weight^T (bf16 in, fp32 sums, bf16 out) on
    torch tensors; a [T, 1024], o_weight [hidden, 1024], y [T, hidden]."""
    import torch

    hidden = _check_oproj(a, o_weight, y, a.device)
    if stream is None:
        stream_ptr = torch.cuda.current_stream(a.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream_ptr = stream.cuda_stream
    else:
        stream_ptr = int(stream)
    st = lib().museattn_oproj(a.data_ptr(), o_weight.data_ptr(), int(a.shape[0]), hidden,
                              y.data_ptr(), stream_ptr)
    if st != OK:
        raise MuseAttnError(st, "museattn_oproj")
    return y


def gather_probe(table, seq_lens, k_cache, v_cache, page_size, max_seq_len, out, work_groups=256,
                 stream=None):
    """museattn_gather_probe on torch tensors: reads every visible key's K and
    V rows of a full-layer step (a memory-system measurement, not the step);
    out: uint32 device tensor of work_groups checksums (int32 storage)."""
    import torch

    for name, t in (("table", table), ("seq_lens", seq_lens), ("k_cache", k_cache),
                    ("v_cache", v_cache), ("out", out)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(table.dtype == torch.int32 and table.dim() == 2, "table must be int32 [B, stride]")
    _need(out.numel() >= work_groups and out.element_size() == 4, "out must hold work_groups uint32")
    if stream is None:
        stream_ptr = torch.cuda.current_stream(table.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream_ptr = stream.cuda_stream
    else:
        stream_ptr = int(stream)
    st = lib().museattn_gather_probe(table.data_ptr(), seq_lens.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), int(page_size), int(seq_lens.shape[0]),
                                     int(table.shape[1]), int(max_seq_len),
                                     int(k_cache.numel() // ROW_BYTES), out.data_ptr(),
                                     int(work_groups), stream_ptr)
    if st != OK:
        raise MuseAttnError(st, "museattn_gather_probe")
    return out
