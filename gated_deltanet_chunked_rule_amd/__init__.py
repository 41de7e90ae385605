"""MI355X-native chunked gated delta rule (GDN linear attention).

Thin Python binding over ``libgdr.so`` (HIP kernels for gfx950 behind the C
ABI declared in ``include/gdr.h``).  This module only marshals arguments:
every step of the computation runs in the library's kernels.  PyTorch is used
for device memory and the current HIP stream.

Functions
---------
``gdr_chunk_fwd`` / ``gdr_chunk_bwd``
    Same names and arguments as the C entry points.
``chunk_gated_delta_rule_fwd`` / ``chunk_gated_delta_rule_bwd``
    The low-level forward/backward pair of the FlashQLA usage listing (curated
    summary "FlashQLA", section "使用方式與需求"): forward returns
    ``(g, A, o, h, final_state)`` and backward ``(dq, dk, dv, db, dg, dh0)``.
    ``h`` (every chunk's entry state) is not exported and is returned as
    ``None``: the backward recomputes it.
``chunk_gated_delta_rule``
    The high-level call of the same listing, differentiable through
    ``torch.autograd``: ``(o, final_state)``.

Layouts: q, k [B, T, Hq, K]; v [B, T, Hv, V]; g, beta [B, T, Hv] fp32;
initial_state [N, Hv, K, V] fp32; cu_seqlens [N + 1] int32 (packed, B = 1).
"""
from __future__ import annotations

import ctypes
import math
import os
from collections import namedtuple
from typing import Optional

import torch

__all__ = ["gdr_chunk_fwd", "gdr_chunk_fwd_noalloc", "gdr_chunk_bwd", "gdr_chunk_fwd_plan", "fwd_workspace_bytes",
           "bwd_workspace_bytes", "chunk_gated_delta_rule",
           "chunk_gated_delta_rule_fwd", "chunk_gated_delta_rule_bwd", "Options", "lib_path",
           "load_library", "GdrError", "timing"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdr.so")
_lib = None

GDR_BF16, GDR_F32 = 0, 1
CP_AUTO, CP_OFF, CP_FORCE = 0, 1, 2


class GdrError(RuntimeError):
    pass


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hv", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("dtype", ctypes.c_int)]


class _Options(ctypes.Structure):
    _fields_ = [("cp_mode", ctypes.c_int), ("cp_segment_chunks", ctypes.c_int32),
                ("cp_warmup_chunks", ctypes.c_int32), ("cp_log_eps", ctypes.c_float),
                ("cp_serial_fallback", ctypes.c_int32), ("precise_vnew", ctypes.c_int32)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_seqs", "total_chunks", "max_chunks", "v_blocks",
                                              "segment_chunks", "warmup_chunks", "total_segments",
                                              "state_workgroups")]


Options = namedtuple("Options", ["cp_mode", "cp_segment_chunks", "cp_warmup_chunks", "cp_log_eps",
                                 "cp_serial_fallback", "precise_vnew"],
                     defaults=[CP_AUTO, 0, 0, 0.0, 0, 0])


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads libgdr.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise GdrError(f"{_LIB_PATH} is missing: build it with "
                       "`python -m gated_deltanet_chunked_rule_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    sp, op = ctypes.POINTER(_Shape), ctypes.POINTER(_Options)
    lib.gdr_chunk_fwd_workspace_size.argtypes = [sp, op, ip]
    lib.gdr_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.gdr_chunk_bwd_workspace_size.argtypes = [sp, op, ip]
    lib.gdr_chunk_bwd_workspace_size.restype = ctypes.c_size_t
    lib.gdr_chunk_fwd.argtypes = [sp, op, vp, vp, vp, fp, fp, ctypes.c_float, fp, ip, ip,
                                  vp, fp, fp, fp, vp, ctypes.c_size_t, vp]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_chunk_bwd.argtypes = [sp, op, vp, vp, vp, fp, fp, fp, vp, fp, ctypes.c_float, fp, ip, ip,
                                  vp, vp, vp, fp, fp, fp, vp, ctypes.c_size_t, vp]
    lib.gdr_chunk_bwd.restype = ctypes.c_int
    lib.gdr_chunk_fwd_noalloc.argtypes = [sp, op, vp, vp, vp, fp, fp, ctypes.c_float, fp, ip, ip,
                                          vp, fp, fp, fp, vp]
    lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdr_chunk_fwd_plan.argtypes = [sp, op, ip, ctypes.POINTER(_PlanInfo)]
    lib.gdr_chunk_fwd_plan.restype = ctypes.c_int
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_timing_enable.argtypes = [ctypes.c_int]
    lib.gdr_timing_enable.restype = None
    lib.gdr_timing_collect.argtypes = []
    lib.gdr_timing_collect.restype = ctypes.c_int
    lib.gdr_timing_entry.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
    lib.gdr_timing_entry.restype = ctypes.c_int
    lib.gdr_timing_reset.argtypes = []
    lib.gdr_timing_reset.restype = None
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise GdrError(f"libgdr status {rc}: {load_library().gdr_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return GDR_BF16
    if dt == torch.float32:
        return GDR_F32
    raise GdrError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _opts(options) -> Optional[_Options]:
    if options is None:
        return None
    o = Options(*options) if not isinstance(options, Options) else options
    return _Options(int(o.cp_mode), int(o.cp_segment_chunks), int(o.cp_warmup_chunks),
                    float(o.cp_log_eps), int(o.cp_serial_fallback), int(o.precise_vnew))


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise GdrError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise GdrError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GdrError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _cu_pair(cu_seqlens, device):
    """(device int32 tensor, host int32 tensor) or (None, None)."""
    if cu_seqlens is None:
        return None, None
    cu = torch.as_tensor(cu_seqlens)
    host = cu.detach().to("cpu", torch.int32).contiguous()
    dev = cu.to(device=device, dtype=torch.int32).contiguous() if not (cu.is_cuda and cu.dtype == torch.int32 and cu.is_contiguous()) else cu
    return dev, host


def _shape(q, v, cu_host):
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    N = (cu_host.numel() - 1) if cu_host is not None else B
    return _Shape(B, T, Hq, Hv, K, V, N, _dtype_code(q.dtype)), N


def _check_shapes(q, k, v, g, beta, N, initial_state=None, A=None, do=None, dht=None):
    """Shape agreement of every tensor argument with q [B,T,Hq,K] and v
    [B,T,Hv,V], checked before anything reaches the library (whose C ABI sees
    bare pointers and would read past a wrongly shaped tensor)."""
    if q.dim() != 4 or v.dim() != 4:
        raise GdrError("q and v must be 4-D: [B, T, Hq, K] and [B, T, Hv, V]")
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    want = {"k": (k, (B, T, Hq, K)), "v": (v, (B, T, Hv, V)), "g": (g, (B, T, Hv)),
            "beta": (beta, (B, T, Hv)), "initial_state": (initial_state, (N, Hv, K, V)),
            "A": (A, (B, T, Hv, 64)), "do": (do, (B, T, Hv, V)), "dht": (dht, (N, Hv, K, V))}
    for name, (t, shape) in want.items():
        if t is not None and tuple(t.shape) != shape:
            raise GdrError(f"shape mismatch: {name} is {tuple(t.shape)}, expected {shape}")


def _host_ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def gdr_chunk_fwd_plan(q, v, cu_seqlens=None, options=None):
    """The planner's choices (segments, warmup, work items) as a dict."""
    lib = load_library()
    _, cu_host = _cu_pair(cu_seqlens, "cpu") if cu_seqlens is not None else (None, None)
    sh, _ = _shape(q, v, cu_host)
    info = _PlanInfo()
    o = _opts(options)
    _check(lib.gdr_chunk_fwd_plan(ctypes.byref(sh), None if o is None else ctypes.byref(o),
                                  _host_ptr(cu_host), ctypes.byref(info)))
    return {n: getattr(info, n) for n, _ in _PlanInfo._fields_}


def fwd_workspace_bytes(q, v, cu_seqlens=None, options=None) -> int:
    """Workspace bytes gdr_chunk_fwd needs (to allocate it once, ahead of time)."""
    lib = load_library()
    _, cu_host = _cu_pair(cu_seqlens, "cpu") if cu_seqlens is not None else (None, None)
    sh, _ = _shape(q, v, cu_host)
    o = _opts(options)
    n = lib.gdr_chunk_fwd_workspace_size(ctypes.byref(sh), None if o is None else ctypes.byref(o),
                                         _host_ptr(cu_host))
    if n == 0:
        _check(-1)
    return n


def bwd_workspace_bytes(q, v, cu_seqlens=None, options=None) -> int:
    """Workspace bytes gdr_chunk_bwd needs."""
    lib = load_library()
    _, cu_host = _cu_pair(cu_seqlens, "cpu") if cu_seqlens is not None else (None, None)
    sh, _ = _shape(q, v, cu_host)
    o = _opts(options)
    n = lib.gdr_chunk_bwd_workspace_size(ctypes.byref(sh), None if o is None else ctypes.byref(o),
                                         _host_ptr(cu_host))
    if n == 0:
        _check(-1)
    return n


def gdr_chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, *,
                  output_final_state=True, output_g_cum=False, output_A=False, options=None,
                  workspace=None, stream=None):
    """Forward chunked prefill.  Returns (o, final_state, g_cum, A); the last
    three are None unless requested."""
    lib = load_library()
    cu_host = None if cu_seqlens is None else torch.as_tensor(cu_seqlens).detach().to("cpu", torch.int32)
    _check_shapes(q, k, v, g, beta, q.shape[0] if cu_host is None else cu_host.numel() - 1,
                  initial_state=initial_state)
    _need(q, "q"); _need(k, "k", q.dtype); _need(v, "v", q.dtype)
    _need(g, "g", torch.float32); _need(beta, "beta", torch.float32)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    dev = q.device
    cu_dev, cu_host = _cu_pair(cu_seqlens, dev)
    sh, N = _shape(q, v, cu_host)
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    scale = K ** -0.5 if scale is None else float(scale)
    o = torch.empty_like(v)
    ht = torch.empty((N, Hv, K, V), device=dev, dtype=torch.float32) if output_final_state else None
    gc = torch.empty((B, T, Hv), device=dev, dtype=torch.float32) if output_g_cum else None
    A = torch.empty((B, T, Hv, 64), device=dev, dtype=torch.float32) if output_A else None
    op = _opts(options)
    opp = None if op is None else ctypes.byref(op)
    ws_bytes = lib.gdr_chunk_fwd_workspace_size(ctypes.byref(sh), opp, _host_ptr(cu_host))
    if ws_bytes == 0:
        _check(-1)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    _check(lib.gdr_chunk_fwd(ctypes.byref(sh), opp, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             ctypes.c_float(scale), _ptr(initial_state), _ptr(cu_dev), _host_ptr(cu_host),
                             _ptr(o), _ptr(ht), _ptr(gc), _ptr(A), _ptr(workspace),
                             ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(st)))
    return o, ht, gc, A


def gdr_chunk_fwd_noalloc(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, *,
                          o=None, final_state=None, output_final_state=True, options=None, stream=None):
    """gdr_chunk_fwd on the library's own device scratch (no workspace): for
    callers that cannot allocate device memory.  Pass preallocated ``o`` (and
    ``final_state``, and cu_seqlens as a device int32 tensor) for a call that
    allocates nothing; missing outputs are allocated here.  Returns
    (o, final_state)."""
    lib = load_library()
    cu_host = None if cu_seqlens is None else torch.as_tensor(cu_seqlens).detach().to("cpu", torch.int32)
    _check_shapes(q, k, v, g, beta, q.shape[0] if cu_host is None else cu_host.numel() - 1,
                  initial_state=initial_state, do=o, dht=final_state)
    _need(q, "q"); _need(k, "k", q.dtype); _need(v, "v", q.dtype)
    _need(g, "g", torch.float32); _need(beta, "beta", torch.float32)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    dev = q.device
    cu_dev, cu_host = _cu_pair(cu_seqlens, dev)
    sh, N = _shape(q, v, cu_host)
    K = q.shape[3]
    scale = K ** -0.5 if scale is None else float(scale)
    o = torch.empty_like(v) if o is None else _need(o, "o", q.dtype)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, v.shape[2], K, v.shape[3]), device=dev, dtype=torch.float32)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32)
    op = _opts(options)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    _check(lib.gdr_chunk_fwd_noalloc(ctypes.byref(sh), None if op is None else ctypes.byref(op), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(g), _ptr(beta), ctypes.c_float(scale),
                                     _ptr(initial_state), _ptr(cu_dev), _host_ptr(cu_host), _ptr(o),
                                     _ptr(final_state), None, None, ctypes.c_void_p(st)))
    return o, final_state


def gdr_chunk_bwd(q, k, v, g, beta, A, do, dht=None, scale=None, initial_state=None,
                  cu_seqlens=None, *, options=None, workspace=None, stream=None):
    """Backward of gdr_chunk_fwd.  Returns (dq, dk, dv, dbeta, dg, dh0)."""
    lib = load_library()
    cu_host = None if cu_seqlens is None else torch.as_tensor(cu_seqlens).detach().to("cpu", torch.int32)
    _check_shapes(q, k, v, g, beta, q.shape[0] if cu_host is None else cu_host.numel() - 1,
                  initial_state=initial_state, A=A, do=do, dht=dht)
    _need(q, "q"); _need(k, "k", q.dtype); _need(v, "v", q.dtype); _need(do, "do", q.dtype)
    _need(g, "g", torch.float32); _need(beta, "beta", torch.float32)
    dev = q.device
    cu_dev, cu_host = _cu_pair(cu_seqlens, dev)
    sh, N = _shape(q, v, cu_host)
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if A is not None:
        _need(A, "A", torch.float32)
    if dht is not None:
        _need(dht, "dht", torch.float32)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    scale = K ** -0.5 if scale is None else float(scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    db = torch.empty_like(beta)
    dg = torch.empty_like(g)
    dh0 = torch.empty((N, Hv, K, V), device=dev, dtype=torch.float32)
    op = _opts(options)
    opp = None if op is None else ctypes.byref(op)
    ws_bytes = lib.gdr_chunk_bwd_workspace_size(ctypes.byref(sh), opp, _host_ptr(cu_host))
    if ws_bytes == 0:
        _check(-1)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    _check(lib.gdr_chunk_bwd(ctypes.byref(sh), opp, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(A), _ptr(do), _ptr(dht), ctypes.c_float(scale), _ptr(initial_state),
                             _ptr(cu_dev), _host_ptr(cu_host), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db),
                             _ptr(dg), _ptr(dh0), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                             ctypes.c_void_p(st)))
    return dq, dk, dv, db, dg, dh0


def chunk_gated_delta_rule_fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                               options=None):
    """(g_cum, A, o, h, final_state) with h = None (not exported)."""
    o, ht, gc, A = gdr_chunk_fwd(q, k, v, g, beta, scale, initial_state, cu_seqlens,
                                 output_final_state=True, output_g_cum=True, output_A=True,
                                 options=options)
    return gc, A, o, None, ht


def chunk_gated_delta_rule_bwd(q, k, v, g, beta, A, do, dht=None, scale=None, initial_state=None,
                               cu_seqlens=None, options=None):
    """(dq, dk, dv, db, dg, dh0); g is the raw log-gate."""
    return gdr_chunk_bwd(q, k, v, g, beta, A, do, dht, scale, initial_state, cu_seqlens,
                         options=options)


class _GDRFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state, scale, cu_seqlens, options):
        # A is not saved: the backward recomputes it (bitwise the same), which is
        # faster than storing and reloading it and keeps 256 B per token and
        # value head out of the saved activations
        o, ht, _, _ = gdr_chunk_fwd(q, k, v, g, beta, scale, initial_state, cu_seqlens,
                                    output_final_state=True, options=options)
        ctx.save_for_backward(q, k, v, g, beta, initial_state)
        ctx.scale, ctx.cu_seqlens, ctx.options = scale, cu_seqlens, options
        return o, ht

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, g, beta, h0 = ctx.saved_tensors
        do = torch.zeros_like(v) if do is None else do.contiguous().to(v.dtype)
        dht = None if dht is None else dht.contiguous().float()
        dq, dk, dv, db, dg, dh0 = gdr_chunk_bwd(q, k, v, g, beta, None, do, dht, ctx.scale, h0,
                                                ctx.cu_seqlens, options=ctx.options)
        return dq, dk, dv, dg, db, (dh0 if h0 is not None else None), None, None, None


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
                           cu_seqlens=None, options=None):
    """High-level call: returns (o, final_state or None); differentiable."""
    scale = q.shape[-1] ** -0.5 if scale is None else float(scale)
    o, ht = _GDRFunction.apply(q, k, v, g, beta, initial_state, scale, cu_seqlens, options)
    return o, (ht if output_final_state else None)


class timing:
    """Per-kernel HIP-event timing of the library's launches (diagnostics)."""

    @staticmethod
    def enable(on: bool = True):
        load_library().gdr_timing_enable(1 if on else 0)

    @staticmethod
    def reset():
        load_library().gdr_timing_reset()

    @staticmethod
    def collect() -> dict:
        lib = load_library()
        n = lib.gdr_timing_collect()
        out = {}
        for i in range(n):
            name, ms, cnt = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int32()
            lib.gdr_timing_entry(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt))
            out[name.value.decode()] = (ms.value, cnt.value)
        return out
