"""Oracle for the chunked gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``gated_deltanet_chunked_rule_amd``) and neither imports the other.

Contents
--------
* ``gdr_fwd`` / ``gdr_bwd``: ctypes front-ends of ``gdr_oracle.c``, the plain
  fp64 token-by-token recurrence of the gated delta rule and its reverse mode
  (the method named "Gated Delta Network (GDN)" on the FlashQLA pages: curated
  summary "FlashQLA" (easyvibecoding.app), sections "中文摘要" and
  "GDN Chunked Prefill的效率問題").  The API shape (q, k, v, g, beta, scale,
  initial_state, cu_seqlens -> o, final_state; backward -> dq, dk, dv, dbeta,
  dg, dh0) follows the usage listing of that page (section "使用方式與需求").
* ``chunk_gcum`` / ``chunk_A``: fp64 NumPy definitions of the two auxiliary
  forward outputs that the low-level forward of that listing returns besides
  ``o``: the processed gate (read as the chunk-local inclusive cumulative sum
  of g) and the per-chunk matrix ``A`` (read as the inverse of the unit lower
  triangular matrix ``I + strict_lower(diag(beta) (D * K K^T))`` with
  ``D_ij = exp(gamma_i - gamma_j)``).  These are definitions written out with a
  library inverse, not the blocked algorithm the kernels use.

Pins (tests/test_oracle_pins.py): brute force with explicit transition
matrices, invariants, closed forms (orthonormal keys, K = 1), central finite
differences of the reverse mode, the gate-decay warmup bound, the delta vectors
of the recurrence against ``chunk_A``, and a hand-derived golden example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import scipy.linalg

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CHUNK = 64  # chunk length of the auxiliary outputs (g_cum, A)


def build(force: bool = True) -> str:
    """Compile gdr_oracle.c into liboracle.so (plain C, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
        lib.oracle_gdr_fwd.argtypes = [i64, ip, i64, i64, i64, i64, dp, dp, dp, dp, dp,
                                       ctypes.c_double, dp, i64, i64, i64, dp, dp, dp, ctypes.c_int]
        lib.oracle_gdr_fwd.restype = ctypes.c_int
        lib.oracle_gdr_bwd.argtypes = [i64, ip, i64, i64, i64, i64, dp, dp, dp, dp, dp,
                                       ctypes.c_double, dp, dp, dp, i64, i64, i64,
                                       dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_gdr_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _flatten(q, k, v, g, beta, cu_seqlens):
    """Turn [B,T,H,D] inputs (or B=1 packed + cu_seqlens) into packed form."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return (q.reshape(B * T, Hq, K), k.reshape(B * T, Hq, K), v.reshape(B * T, Hv, V),
            g.reshape(B * T, Hv), beta.reshape(B * T, Hv), cu, (B, T, Hq, Hv, K, V))


def gdr_fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, *,
            heads=None, t_max=0, want_u=False, threads=None):
    """fp64 token recurrence.

    Returns ``(o [B,T,Hv,V], final_state [N,Hv,K,V])`` (plus ``u`` when
    ``want_u``).  ``heads=(h0, h1)`` restricts the work to value heads
    ``[h0, h1)`` (other heads are returned as NaN); ``t_max > 0`` processes
    only the first ``t_max`` tokens of every sequence (later outputs NaN).
    """
    qf, kf, vf, gf, bf, cu, (B, T, Hq, Hv, K, V) = _flatten(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = K ** -0.5
    h0 = _f64(initial_state)
    if h0 is not None:
        h0 = h0.reshape(N, Hv, K, V)
    hb, he = (0, Hv) if heads is None else heads
    o = np.full((B * T, Hv, V), np.nan)
    ht = np.full((N, Hv, K, V), np.nan)
    u = np.full((B * T, Hv, V), np.nan) if want_u else None
    rc = _load().oracle_gdr_fwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), Hq, Hv, K, V,
                                _ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf), float(scale),
                                _ptr(h0), int(t_max), hb, he, _ptr(o), _ptr(ht), _ptr(u),
                                threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gdr_fwd failed ({rc})")
    o = o.reshape(B, T, Hv, V)
    if want_u:
        return o, ht, u.reshape(B, T, Hv, V)
    return o, ht


def gdr_bwd(q, k, v, g, beta, do, dht=None, scale=None, initial_state=None, cu_seqlens=None,
            *, qk_heads=None, t_max=0, threads=None):
    """Reverse mode of ``gdr_fwd`` for the loss <o, do> + <final_state, dht>.

    Returns ``(dq, dk, dv, dbeta, dg, dh0)`` with the layouts of q, k, v, beta,
    g and initial_state.  dg is the gradient with respect to the raw per-token
    log-gate g.  ``qk_heads=(a, b)`` restricts to q/k heads [a, b) and their
    value heads (other entries NaN).
    """
    qf, kf, vf, gf, bf, cu, (B, T, Hq, Hv, K, V) = _flatten(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = K ** -0.5
    h0 = _f64(initial_state)
    if h0 is not None:
        h0 = h0.reshape(N, Hv, K, V)
    dof = _f64(do).reshape(B * T, Hv, V)
    dhtf = None if dht is None else _f64(dht).reshape(N, Hv, K, V)
    hb, he = (0, Hq) if qk_heads is None else qk_heads
    dq = np.zeros((B * T, Hq, K))
    dk = np.zeros((B * T, Hq, K))
    dv = np.full((B * T, Hv, V), np.nan)
    db = np.full((B * T, Hv), np.nan)
    dg = np.full((B * T, Hv), np.nan)
    dh0 = np.full((N, Hv, K, V), np.nan)
    rc = _load().oracle_gdr_bwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), Hq, Hv, K, V,
                                _ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf), float(scale),
                                _ptr(h0), _ptr(dof), _ptr(dhtf), int(t_max), hb, he,
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db), _ptr(dg), _ptr(dh0),
                                threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gdr_bwd failed ({rc})")
    if qk_heads is not None:
        mask = np.ones(Hq, bool)
        mask[hb:he] = False
        dq[:, mask] = np.nan
        dk[:, mask] = np.nan
    return (dq.reshape(B, T, Hq, K), dk.reshape(B, T, Hq, K), dv.reshape(B, T, Hv, V),
            db.reshape(B, T, Hv), dg.reshape(B, T, Hv), dh0)


def _chunks(cu):
    """(start, stop) token ranges of the CHUNK-token chunks of every sequence;
    chunks restart at every sequence start and the last one may be short."""
    out = []
    for n in range(len(cu) - 1):
        for s in range(int(cu[n]), int(cu[n + 1]), CHUNK):
            out.append((s, min(s + CHUNK, int(cu[n + 1]))))
    return out


def chunk_gcum(g, cu_seqlens=None):
    """Chunk-local inclusive cumulative sum of the log-gate g [B,T,Hv] (fp64)."""
    g = _f64(g)
    B, T, Hv = g.shape
    cu = np.arange(B + 1) * T if cu_seqlens is None else np.asarray(cu_seqlens)
    gf = g.reshape(B * T, Hv)
    out = np.empty_like(gf)
    for s, e in _chunks(cu):
        out[s:e] = np.cumsum(gf[s:e], axis=0)
    return out.reshape(B, T, Hv)


def chunk_A(k, g, beta, Hv, cu_seqlens=None):
    """Per-chunk A = (I + L)^-1 with L_ij = beta_i exp(gamma_i - gamma_j) k_i.k_j
    for i > j (zero elsewhere), gamma the chunk-local cumsum of g.

    Returned as [B, T, Hv, CHUNK]: the row of A belonging to token t of its
    chunk; columns beyond the chunk's length are zero.
    """
    k, g, beta = _f64(k), _f64(g), _f64(beta)
    B, T, Hq, K = k.shape
    G = Hv // Hq
    cu = np.arange(B + 1) * T if cu_seqlens is None else np.asarray(cu_seqlens)
    kf = k.reshape(B * T, Hq, K)
    gam = chunk_gcum(g, cu_seqlens).reshape(B * T, Hv)
    bf = beta.reshape(B * T, Hv)
    out = np.zeros((B * T, Hv, CHUNK))
    for s, e in _chunks(cu):
        n = e - s
        for h in range(Hv):
            kc = kf[s:e, h // G]
            gm = gam[s:e, h]
            L = np.tril(bf[s:e, h][:, None] * np.exp(gm[:, None] - gm[None, :]) * (kc @ kc.T), -1)
            out[s:e, h, :n] = scipy.linalg.solve_triangular(np.eye(n) + L, np.eye(n), lower=True,
                                                            unit_diagonal=True)
    return out.reshape(B, T, Hv, CHUNK)
