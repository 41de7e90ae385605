"""Seeded synthetic inputs for the chunked gated delta rule.

This module holds no arithmetic of the method itself: it only draws random
tensors with the shapes and distributions of the five workloads (and of
smaller test cases) and rounds them to the working precision.  Both the HIP
path's tests/benchmark and the oracle consume exactly the tensors it returns.

Recipe (NumPy PCG64, ``np.random.default_rng(seed)``), in this draw order:
  1. varlen lengths (when the workload is packed), 2. q, 3. k, 4. v, 5. g,
  6. beta, 7. initial_state, 8. do, 9. dht, 10. the permutation that picks
  the non-decaying value heads (mixed-gate workloads only).
* q, k ~ N(0, 1), L2-normalised per (token, head) vector in fp32, then cast.
* v ~ N(0, 1).
* g = log(U(a, b)) per (token, value head); in mixed-gate workloads a seeded
  30 % of the value heads (round(0.3 Hv)) use g = 0 instead.
* beta = sigmoid(N(0, 1)).
* initial_state, dht ~ N(0, 0.02^2) fp32;  do ~ N(0, 1).
* bf16 workloads round q, k, v, do to bfloat16 (round to nearest even);
  g, beta and the states stay fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hv: int
    K: int
    V: int
    dtype: str                       # "bf16" or "f32"
    seed: int
    gate: Tuple[float, float] = (0.85, 1.0)
    zero_gate_frac: float = 0.0      # fraction of value heads with g == 0
    initial_state: bool = False
    varlen: Optional[dict] = None    # {"n": N, "lo": lo, "hi": hi} (B must be 1)
    backward: bool = False
    description: str = ""
    chunk: int = 64


# The five workloads.  Sizes, dtypes and distributions follow the workload
# descriptions; for the varlen and long-context ones the gate and beta draws
# are those of the tiny workload (log U(0.85, 1), sigmoid(N(0,1))).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 2, 2, 32, 32, "f32", 1,
                          description="tiny forward, fp32, T=256, H=2, K=V=32"),
    "edge_prefill": Workload("edge_prefill", 1, 8192, 16, 32, 128, 128, "bf16", 2,
                             gate=(0.9, 0.999), zero_gate_frac=0.3, initial_state=True,
                             description="edge prefill, bf16, T=8192, Hq=16, Hv=32, 30% g=0 heads"),
    "long_context": Workload("long_context", 1, 65536, 4, 8, 128, 128, "bf16", 3,
                             description="long context, bf16, B=1, T=65536, Hq=4, Hv=8"),
    "varlen": Workload("varlen", 1, 131072, 16, 64, 128, 128, "bf16", 4, initial_state=True,
                       varlen={"n": 16, "lo": 512, "hi": 32768},
                       description="16 packed sequences, log-uniform lengths, T=131072, Hv=64"),
    "backward": Workload("backward", 2, 16384, 16, 32, 128, 128, "bf16", 5, backward=True,
                         description="backward, bf16, B=2, T=16384, Hq=16, Hv=32"),
}


def varlen_lengths(rng: np.random.Generator, n: int, lo: int, hi: int, total: int) -> np.ndarray:
    """n lengths log-uniform in [lo, hi], rescaled (with clamping) to sum to total."""
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    for _ in range(200):
        x = np.clip(x * (total / x.sum()), lo, hi)
        if abs(x.sum() - total) < 0.5:
            break
    L = np.floor(x).astype(np.int64)
    rem = int(total - L.sum())
    order = np.argsort(-L)
    i = 0
    while rem != 0 and i < 10 * n:
        j = order[i % n]
        step = 1 if rem > 0 else -1
        if lo <= L[j] + step <= hi:
            L[j] += step
            rem -= step
        i += 1
    if L.sum() != total:
        raise ValueError("cannot meet the requested total with these bounds")
    return L


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def _l2norm(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def make_inputs(w: Workload, T: Optional[int] = None, with_grads: Optional[bool] = None) -> dict:
    """Draw the inputs of workload ``w`` (optionally with T overridden).

    Returns a dict of CPU torch tensors: q, k, v (working dtype), g, beta
    (fp32), initial_state (fp32 or None), cu_seqlens (int32 or None), do, dht
    (when gradients are requested), plus ``scale`` and ``workload``.
    """
    rng = np.random.default_rng(w.seed)
    T = w.T if T is None else T
    B, Hq, Hv, K, V = w.B, w.Hq, w.Hv, w.K, w.V
    cu = None
    N = B
    if w.varlen is not None:
        if B != 1:
            raise ValueError("packed workloads use B == 1")
        lens = varlen_lengths(rng, w.varlen["n"], w.varlen["lo"], w.varlen["hi"], T)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        N = len(lens)
    q = _l2norm(_normal(rng, (B, T, Hq, K)))
    k = _l2norm(_normal(rng, (B, T, Hq, K)))
    v = _normal(rng, (B, T, Hv, V))
    a, b = w.gate
    g = np.log(rng.uniform(a, b, size=(B, T, Hv))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-_normal(rng, (B, T, Hv))))).astype(np.float32)
    h0 = _normal(rng, (N, Hv, K, V), 0.02) if w.initial_state else None
    grads = w.backward if with_grads is None else with_grads
    do = _normal(rng, (B, T, Hv, V)) if grads else None
    dht = _normal(rng, (N, Hv, K, V), 0.02) if grads else None
    if w.zero_gate_frac > 0:
        nz = int(round(w.zero_gate_frac * Hv))
        zero_heads = rng.permutation(Hv)[:nz]
        g[:, :, zero_heads] = 0.0
    out = {
        "q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
        "g": torch.from_numpy(g), "beta": torch.from_numpy(beta),
        "initial_state": None if h0 is None else torch.from_numpy(h0),
        "cu_seqlens": None if cu is None else torch.from_numpy(cu),
        "do": None if do is None else _cast(do, w.dtype),
        "dht": None if dht is None else torch.from_numpy(dht),
        "scale": K ** -0.5,
        "workload": w,
    }
    return out


def custom(name="custom", *, B=1, T=256, Hq=2, Hv=2, K=32, V=32, dtype="f32", seed=0,
           gate=(0.85, 1.0), zero_gate_frac=0.0, initial_state=False, varlen=None,
           backward=False) -> Workload:
    """A workload of arbitrary size with the same recipe (used by tests)."""
    return Workload(name, B, T, Hq, Hv, K, V, dtype, seed, gate=gate,
                    zero_gate_frac=zero_gate_frac, initial_state=initial_state,
                    varlen=varlen, backward=backward)


def packed_from_lengths(w: Workload, lengths) -> dict:
    """Inputs of workload w (B=1) packed from explicit sequence lengths."""
    T = int(sum(lengths))
    base = make_inputs(Workload(w.name, 1, T, w.Hq, w.Hv, w.K, w.V, w.dtype, w.seed,
                                gate=w.gate, zero_gate_frac=w.zero_gate_frac,
                                initial_state=False, backward=w.backward))
    rng = np.random.default_rng(w.seed + 1000)
    N = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    base["cu_seqlens"] = torch.from_numpy(cu)
    base["initial_state"] = (torch.from_numpy(_normal(rng, (N, w.Hv, w.K, w.V), 0.02))
                             if w.initial_state else None)
    if base["dht"] is not None:
        base["dht"] = torch.from_numpy(_normal(rng, (N, w.Hv, w.K, w.V), 0.02))
    return base
