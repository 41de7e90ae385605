"""The no-allocation forward entry point (gdr_chunk_fwd_noalloc, for callers
that cannot allocate device memory) against gdr_chunk_fwd on the same inputs.

Both run the same kernels; only the workspace differs (the library's own
per-device scratch instead of a caller buffer), so the outputs must agree
bitwise.  Two calls in a row, the second smaller, show that what the first
leaves in the shared scratch does not leak into the second."""
import pytest
import torch

import gated_deltanet_chunked_rule_amd as gdr
import gdr_inputs as gi
from parity import dev

pytestmark = pytest.mark.gpu


def _both(inp, options=None):
    q, k, v, g, b, h0 = (dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "initial_state"))
    cu = inp["cu_seqlens"]
    cu_d = None if cu is None else dev(cu)
    o_ref, ht_ref, _, _ = gdr.gdr_chunk_fwd(q, k, v, g, b, inp["scale"], h0, cu_d, options=options)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    o, ht = gdr.gdr_chunk_fwd_noalloc(q, k, v, g, b, inp["scale"], h0, cu_d, o=o, final_state=ht,
                                      options=options)
    torch.cuda.synchronize()
    return o_ref, ht_ref, o, ht


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: the long-context shape (114 MiB of the 128 MiB scratch, CP
    # segments); second: a smaller packed call with exact segments for g = 0
    # heads (transition and scan buffers at other offsets of the scratch)
    big = gi.make_inputs(gi.WORKLOADS["long_context"])
    print("[noalloc] call 1: long-context shape", flush=True)
    o_ref, ht_ref, o, ht = _both(big)
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
    w = gi.custom(B=1, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=97, initial_state=True,
                  gate=(0.9, 0.999), zero_gate_frac=0.5)
    small = gi.packed_from_lengths(w, [64 * 9 + 7, 1, 64 * 3, 0, 64 * 6 + 40])
    print("[noalloc] call 2: small packed call, forced CP", flush=True)
    o_ref, ht_ref, o, ht = _both(small, gdr.Options(gdr.CP_FORCE, 2, 1))
    assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
