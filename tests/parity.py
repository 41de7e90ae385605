"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
(via the Python binding) and the fp64 oracle on the same seeded inputs, and
compare with err(x) = max|x - ref| / max|ref| per output tensor."""
from __future__ import annotations

import numpy as np
import torch

import gated_deltanet_chunked_rule_amd as gdr
import oracle

# Tolerances on err(x): bf16 inputs 2e-2 (o and gradients) and 1e-2
# (final_state); fp32 inputs 1e-4 for every output.
TOL = {"bf16": {"o": 2e-2, "final_state": 1e-2, "grad": 2e-2, "dh0": 1e-2},
       "f32": {"o": 1e-4, "final_state": 1e-4, "grad": 1e-4, "dh0": 1e-4}}


def dev(x, device="cuda"):
    return None if x is None else x.to(device).contiguous()


def f64(x):
    return None if x is None else x.detach().to("cpu", torch.float64).numpy()


def rel_err(x, ref):
    x = f64(x) if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    assert m.any()
    denom = np.max(np.abs(ref[m]))
    if denom == 0:
        return float(np.max(np.abs(x[m])))
    return float(np.max(np.abs(x[m] - ref[m])) / denom)


def gpu_fwd(inp, options=None, **kw):
    return gdr.gdr_chunk_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]),
                             dev(inp["beta"]), inp["scale"], dev(inp["initial_state"]),
                             inp["cu_seqlens"], options=options, **kw)


def oracle_fwd(inp, heads=None, t_max=0):
    return oracle.gdr_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                          f64(inp["beta"]), inp["scale"], f64(inp["initial_state"]),
                          None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy(),
                          heads=heads, t_max=t_max)


def gpu_bwd(inp, A=None, options=None):
    return gdr.gdr_chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]),
                             dev(inp["beta"]), A, dev(inp["do"]), dev(inp["dht"]), inp["scale"],
                             dev(inp["initial_state"]), inp["cu_seqlens"], options=options)


def oracle_bwd(inp, qk_heads=None):
    return oracle.gdr_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                          f64(inp["beta"]), f64(inp["do"]), f64(inp["dht"]), inp["scale"],
                          f64(inp["initial_state"]),
                          None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy(),
                          qk_heads=qk_heads)


def head_slice(x, lo, hi, axis):
    idx = [slice(None)] * x.ndim
    idx[axis] = slice(lo, hi)
    return x[tuple(idx)]


def set_chunk_gate_mass(inp, mass_of_chunk, chunk=64):
    """Replace g by a per-chunk constant: every token of chunk c gets
    mass_of_chunk(c) / chunk, so each full chunk's gate sum is mass_of_chunk(c)."""
    g = inp["g"].clone()
    T = g.shape[1]
    for c in range((T + chunk - 1) // chunk):
        g[:, c * chunk:(c + 1) * chunk, :] = mass_of_chunk(c) / chunk
    inp["g"] = g
    return inp


# Per-value-head gate mass per full chunk; with ln(1e-6) the shortest warmup
# is 7, 3, -, 1, 5, 2, -, 6 chunks (two heads would need more than 8 and take
# the exact path), so the heads of one q/k group start their segments at
# different chunks.
HEAD_MASS = (2.0, 5.0, 1.5, 14.0, 3.0, 7.0, 0.5, 2.5)


def head_mass_inputs(backward=False):
    import gdr_inputs as gi
    w = gi.custom(B=1, Hq=2, Hv=8, K=128, V=128, dtype="bf16", seed=46, initial_state=True, backward=backward)
    inp = gi.packed_from_lengths(w, [64 * 9 + 7, 64 * 5, 64 * 12 + 3, 30])
    g = torch.empty_like(inp["g"])
    for h, m in enumerate(HEAD_MASS):
        g[..., h] = -m / 64
    inp["g"] = g
    return inp
