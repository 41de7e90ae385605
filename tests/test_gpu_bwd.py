"""Backward parity of the HIP path (through the C ABI) against the oracle's
reverse mode (the token recurrence differentiated step by step).

Metric: err(x) = max|x - ref| / max|ref| per gradient; bf16 workloads must
reach 2e-2 on dq, dk, dv, dbeta, dg and 1e-2 on dh0, fp32 workloads 1e-4."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_rule_amd as gdr
import gdr_inputs as gi
from parity import (TOL, dev, f64, gpu_bwd, gpu_fwd, head_mass_inputs, oracle_bwd, oracle_fwd, rel_err,
                    set_chunk_gate_mass)

pytestmark = pytest.mark.gpu
NAMES = ["dq", "dk", "dv", "dbeta", "dg", "dh0"]


def check_bwd(inp, qk_heads=None, label="", A=None, options=None):
    w = inp["workload"]
    print(f"[bwd] {label or w.name} B={w.B} T={inp['q'].shape[1]} Hq={w.Hq} Hv={w.Hv} K={w.K} {w.dtype}",
          flush=True)
    grads = gpu_bwd(inp, A=A, options=options)
    torch.cuda.synchronize()
    ref = oracle_bwd(inp, qk_heads=qk_heads)
    tol = TOL[w.dtype]
    errs = {}
    for name, x, r in zip(NAMES, grads, ref):
        if qk_heads is not None and name in ("dv", "dbeta", "dg", "dh0"):
            G = w.Hv // w.Hq
            axis = 2 if name != "dh0" else 1
            lo, hi = qk_heads[0] * G, qk_heads[1] * G
            mask = np.zeros(r.shape[axis], bool)
            mask[lo:hi] = True
            r = np.where(np.expand_dims(mask, tuple(i for i in range(r.ndim) if i != axis)), r, np.nan)
        errs[name] = rel_err(x, r)
    print("      " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()), flush=True)
    for name, e in errs.items():
        bound = tol["dh0"] if name == "dh0" else tol["grad"]
        assert np.isfinite(e) and e <= bound, (name, e)
    return grads


@pytest.mark.parametrize("K", [32, 64, 128])
def test_ragged_bf16(K):
    w = gi.custom(B=2, T=64 * 3 + 29, Hq=2, Hv=4, K=K, V=K, dtype="bf16", seed=70, initial_state=True,
                  backward=True)
    check_bwd(gi.make_inputs(w))


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("bf16", 64), ("f32", 32)])
def test_strong_decay_gates_backward(dtype, K):
    # gates alpha = e^g in (1e-6, 1e-2): e^gamma underflows fp32 within a
    # chunk; the gradients' decay factors must come from differences of gamma
    w = gi.custom(B=1, T=64 * 4 + 21, Hq=2, Hv=4, K=K, V=K, dtype=dtype, seed=48, initial_state=True,
                  gate=(1e-6, 1e-2), backward=True)
    check_bwd(gi.make_inputs(w), label=f"strong decay {dtype} K={K}")


def test_backward_one_head_131072_tokens():
    # one value head over 2048 chunks: the states and reverse passes split
    # it into many CP segments, each warming up before its start (states)
    # and after its end (reverse pass)
    w = gi.custom(B=1, T=131072, Hq=1, Hv=1, K=128, V=128, dtype="bf16", seed=51, initial_state=True,
                  backward=True)
    inp = gi.make_inputs(w)
    info = gdr.gdr_chunk_fwd_plan(dev(inp["q"]), dev(inp["v"]))
    print(f"      plan: {info}", flush=True)
    assert info["total_segments"] >= 64
    check_bwd(inp, label="one head, 131072 tokens")


def test_odd_head_counts_and_many_short_rows_backward():
    # three q/k heads (six value heads) and 24 rows of 70 tokens
    w = gi.custom(B=24, T=70, Hq=3, Hv=6, K=128, V=128, dtype="bf16", seed=50, initial_state=True,
                  backward=True)
    check_bwd(gi.make_inputs(w), label="Hq=3 Hv=6 B=24")


def test_fp32_k32():
    w = gi.custom(B=1, T=64 * 4 + 7, Hq=2, Hv=2, K=32, V=32, dtype="f32", seed=71, initial_state=True,
                  backward=True)
    check_bwd(gi.make_inputs(w))


def test_fp32_tiny_workload_backward():
    w = gi.WORKLOADS["tiny_fp32"]
    inp = gi.make_inputs(w, with_grads=True)
    check_bwd(inp)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_grouped_heads(G):
    w = gi.custom(B=1, T=200, Hq=2, Hv=2 * G, K=128, V=128, dtype="bf16", seed=72 + G, backward=True)
    check_bwd(gi.make_inputs(w))


def test_varlen_with_empty_sequences():
    w = gi.custom(B=1, Hq=2, Hv=4, K=64, V=64, dtype="bf16", seed=74, initial_state=True, backward=True)
    check_bwd(gi.packed_from_lengths(w, [65, 0, 1, 130, 64]))


def test_zero_gate_heads_and_no_state_terms():
    w = gi.custom(B=1, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=75, backward=True,
                  gate=(0.9, 0.999), zero_gate_frac=0.5)
    inp = gi.make_inputs(w)
    inp["dht"] = None
    check_bwd(inp)


def test_supplied_A_equals_recomputed():
    w = gi.custom(B=1, T=64 * 3 + 5, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=76, initial_state=True,
                  backward=True)
    inp = gi.make_inputs(w)
    _, _, _, A = gpu_fwd(inp, output_A=True)
    g1 = gpu_bwd(inp)
    g2 = gpu_bwd(inp, A=A)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_autograd_wrapper_matches_entry_point():
    w = gi.custom(B=1, T=150, Hq=1, Hv=2, K=64, V=64, dtype="bf16", seed=77, initial_state=True,
                  backward=True)
    inp = gi.make_inputs(w)
    q, k, v, g, b, h0 = (dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "initial_state"))
    for t in (q, k, v, g, b, h0):
        t.requires_grad_(True)
    o, ht = gdr.chunk_gated_delta_rule(q, k, v, g, b, inp["scale"], h0, output_final_state=True)
    do, dht = dev(inp["do"]), dev(inp["dht"])
    grads = torch.autograd.grad([o, ht], [q, k, v, b, g, h0], [do, dht])
    ref = gpu_bwd(inp)
    for a, r in zip(grads, ref):
        assert torch.equal(a, r)


def test_deterministic():
    w = gi.custom(B=1, T=64 * 5 + 3, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=78, initial_state=True,
                  backward=True)
    inp = gi.make_inputs(w)
    g1 = gpu_bwd(inp)
    g2 = gpu_bwd(inp)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_workload_full_size_all_heads():
    # the backward workload (B=2, T=16384, Hq=16, Hv=32) with every head
    # compared: dq, dk, dv, dbeta, dg, dh0 element by element
    inp = gi.make_inputs(gi.WORKLOADS["backward"])
    check_bwd(inp, label="backward workload, all heads")


def _autograd_vs_oracle(inp, label):
    # o, final_state and the gradients of <o, do> + <final_state, dht> through
    # the differentiable wrapper (the training-step path: forward, autograd,
    # backward with A recomputed), against the oracle's recurrence and reverse
    # mode on the same inputs
    w = inp["workload"]
    print(f"[autograd] {label} T={inp['q'].shape[1]} Hq={w.Hq} Hv={w.Hv} B={w.B}", flush=True)
    leaves = [dev(inp[n]).requires_grad_(True) for n in ("q", "k", "v", "g", "beta")]
    h0 = dev(inp["initial_state"])
    if h0 is not None:
        h0.requires_grad_(True)
    cu = inp["cu_seqlens"]
    o, ht = gdr.chunk_gated_delta_rule(*leaves, inp["scale"], h0, output_final_state=True,
                                       cu_seqlens=None if cu is None else dev(cu))
    wrt = leaves + ([h0] if h0 is not None else [])
    grads = torch.autograd.grad([o, ht], wrt, [dev(inp["do"]), dev(inp["dht"])])
    torch.cuda.synchronize()
    ro, rht = oracle_fwd(inp)
    rdq, rdk, rdv, rdb, rdg, rdh0 = oracle_bwd(inp)
    errs = {"o": rel_err(o.detach(), ro), "final_state": rel_err(ht.detach(), rht)}
    for name, x, r in zip(("dq", "dk", "dv", "dg", "dbeta"), grads, (rdq, rdk, rdv, rdg, rdb)):
        errs[name] = rel_err(x, r)
    if h0 is not None:
        errs["dh0"] = rel_err(grads[5], rdh0)
    print("      " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()), flush=True)
    for name, e in errs.items():
        bound = TOL["bf16"]["o"] if name == "o" else TOL["bf16"]["grad"]
        if name in ("final_state", "dh0"):
            bound = TOL["bf16"]["final_state"]
        assert np.isfinite(e) and e <= bound, (name, e)


def test_training_step_through_autograd_matches_oracle():
    # one training-step shape of the value-head sweep (Hv = 24, the TP-style
    # share; Hq = Hv / 2; two 8192-token sequences; no initial state)
    w = gi.custom(B=2, T=8192, Hq=12, Hv=24, K=128, V=128, dtype="bf16", seed=95, backward=True)
    _autograd_vs_oracle(gi.make_inputs(w), "sweep shape Hv=24")


def test_training_step_through_autograd_packed_with_state():
    # Hv = 48 with packed sequences of unequal length and per-sequence initial
    # states (dh0 through autograd)
    w = gi.custom(B=1, Hq=24, Hv=48, K=128, V=128, dtype="bf16", seed=96, initial_state=True, backward=True)
    _autograd_vs_oracle(gi.packed_from_lengths(w, [3000, 4096, 96, 1000]), "packed Hv=48")


def test_certificate_excludes_positive_gates_and_expanding_keys_backward():
    # As in the forward test: fast decay (-7.5 per chunk) would certify every
    # head on 2-chunk windows, before each segment start (chunks 4-5, 10-11)
    # and after each segment end (chunks 6-7, 12-13); head 1 has g > 0 and
    # head 2 one beta |k|^2 = 3 token in chunks 8-9, inside no window.  With
    # the serial fallback those heads run whole in both serial passes, so
    # their gradients equal the unsegmented call's bitwise (G = 1: dq and dk
    # of a q/k head come from its one value head), while a certified head's
    # per-token gradients next to a segment boundary carry the warmup error.
    w = gi.custom(B=1, T=64 * 16 + 9, Hq=4, Hv=4, K=128, V=128, dtype="bf16", seed=48, initial_state=True,
                  backward=True)
    inp = set_chunk_gate_mass(gi.make_inputs(w), lambda c: -7.5)
    g, beta = inp["g"].clone(), inp["beta"].clone()
    g[0, 8 * 64 + 10:8 * 64 + 13, 1] = 0.2
    beta[0, 9 * 64 + 20, 2] = 3.0
    inp["g"], inp["beta"] = g, beta
    check_bwd(inp, options=gdr.Options(gdr.CP_FORCE, 6, 2), label="g > 0 and beta |k|^2 > 2 in segment bodies")
    off = gpu_bwd(inp, options=gdr.Options(gdr.CP_OFF))
    ser = gpu_bwd(inp, options=gdr.Options(gdr.CP_FORCE, 6, 2, 0.0, 1))
    torch.cuda.synchronize()
    for h in (1, 2):
        for name, a, b in zip(NAMES, ser, off):
            x, y = (a[:, h], b[:, h]) if name == "dh0" else (a[:, :, h], b[:, :, h])
            assert torch.equal(x, y), (name, h)
    for h in (0, 3):   # fp32 dg and dbeta of a certified head differ somewhere
        assert not (torch.equal(ser[4][:, :, h], off[4][:, :, h]) and torch.equal(ser[3][:, :, h], off[3][:, :, h])), h


# CP segments in the backward (bf16): both serial passes (the recomputed
# chunk states and the reverse pass over the state gradient) run per segment.

@pytest.mark.parametrize("K", [64, 128])
def test_cp_segments_mixed_heads(K):
    # Half the heads decay fast enough for a 2-chunk warmup to certify, both
    # before each segment start and after each segment end; the g = 0 heads
    # take the exact path in both passes (transitions, scans, exact starts).
    w = gi.custom(B=2, T=64 * 11 + 23, Hq=2, Hv=4, K=K, V=K, dtype="bf16", seed=90, initial_state=True,
                  backward=True, gate=(0.5, 0.8), zero_gate_frac=0.5)
    check_bwd(gi.make_inputs(w), options=gdr.Options(gdr.CP_FORCE, 3, 2), label=f"CP mixed heads K={K}")


@pytest.mark.parametrize("seg", [1, 4])
def test_cp_exact_segments_all_uncertified(seg):
    w = gi.custom(B=1, T=64 * 9 + 5, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=91, initial_state=True,
                  backward=True, zero_gate_frac=1.0)
    check_bwd(gi.make_inputs(w), options=gdr.Options(gdr.CP_FORCE, seg, 2), label=f"CP exact L={seg}")


def test_cp_serial_fallback_backward():
    w = gi.custom(B=1, T=64 * 14 + 5, Hq=2, Hv=8, K=128, V=128, dtype="bf16", seed=92, initial_state=True,
                  backward=True, gate=(0.9, 0.999), zero_gate_frac=0.5)
    inp = gi.make_inputs(w)
    g1 = check_bwd(inp, options=gdr.Options(gdr.CP_FORCE, 4, 2, 0.0, 1), label="CP serial fallback")
    g2 = check_bwd(inp, options=gdr.Options(gdr.CP_FORCE, 4, 2, 0.0, 0), label="CP exact segments")
    for a, b in zip(g1, g2):   # the same recurrence up to rounding order
        assert rel_err(a, f64(b)) <= 2e-2


def test_cp_backward_varlen():
    w = gi.custom(B=1, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=93, initial_state=True, backward=True,
                  gate=(0.5, 0.8), zero_gate_frac=0.5)
    inp = gi.packed_from_lengths(w, [64 * 9 + 7, 1, 64 * 3, 0, 64 * 6 + 40])
    check_bwd(inp, options=gdr.Options(gdr.CP_FORCE, 2, 1), label="CP varlen")


def test_many_chunks_per_workgroup():
    # Enough (chunk, query/key head) items that each workgroup of the
    # persistent per-chunk gradient kernel walks several of them, crossing
    # chunk and head boundaries; sampled heads keep the oracle fast.
    w = gi.custom(B=1, T=64 * 600 + 17, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=94, initial_state=True,
                  backward=True, gate=(0.9, 0.999))
    check_bwd(gi.make_inputs(w), qk_heads=(1, 2), label="many chunks per workgroup")


def test_short_warmup_takes_enough_chunks_backward():
    # Gate masses repeating (-0.5, -20, -1) per chunk: both the state pass
    # (chunks before a segment start) and the reverse pass (chunks after a
    # segment end) need exactly two warmup chunks; one leaves e^-1 or e^-0.5.
    w = gi.custom(B=1, T=64 * 12 + 5, Hq=1, Hv=2, K=128, V=128, dtype="bf16", seed=44, initial_state=True,
                  backward=True)
    inp = set_chunk_gate_mass(gi.make_inputs(w), lambda c: (-0.5, -20.0, -1.0)[c % 3])
    check_bwd(inp, options=gdr.Options(gdr.CP_FORCE, 3, 4), label="stepped gates, warmup <= 4")
    ref = oracle_bwd(inp)
    loose = gpu_bwd(inp, options=gdr.Options(gdr.CP_FORCE, 3, 1, -0.1))
    torch.cuda.synchronize()
    assert max(rel_err(x, r) for x, r in zip(loose, ref)) > 5e-2


def test_warmup_length_differs_per_head_varlen_backward():
    # per-value-head gate masses (shortest warmups 7, 3, -, 1, 5, 2, -, 6
    # chunks; two heads exact), packed sequences, four value heads per q/k head
    check_bwd(head_mass_inputs(backward=True), options=gdr.Options(gdr.CP_FORCE, 3, 8),
              label="per-head warmups, varlen, G=4")


@pytest.mark.parametrize("K", [64, 128])
def test_workspace_filled_with_nan(K):
    # Every workspace element the backward reads (A with its zero blocks above
    # the diagonal, the chunk states, Vnew, ...) is written before it is read:
    # a workspace filled with NaN bit patterns gives the same gradients.
    w = gi.custom(B=1, T=64 * 2 + 8, Hq=2, Hv=2, K=K, V=K, dtype="bf16", seed=76, backward=True)
    inp = gi.make_inputs(w)
    nbytes = gdr.bwd_workspace_bytes(dev(inp["q"]), dev(inp["v"]))
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    print(f"[bwd] NaN-filled workspace K={K} T={w.T}", flush=True)
    grads = gdr.gdr_chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                              None, dev(inp["do"]), dev(inp["dht"]), inp["scale"], None, None, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle_bwd(inp)
    for name, x, r in zip(NAMES, grads, ref):
        e = rel_err(x, r)
        bound = TOL["bf16"]["dh0"] if name == "dh0" else TOL["bf16"]["grad"]
        assert np.isfinite(e) and e <= bound, (name, e)


def test_empty_sequence_gradient_passes_through():
    # with no token the final-state gradient reaches the initial state unchanged
    w = gi.custom(B=2, T=0, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=81, initial_state=True, backward=True)
    inp = gi.make_inputs(w)
    print("[bwd] T=0", flush=True)
    grads = gpu_bwd(inp)
    torch.cuda.synchronize()
    assert all(x.numel() == 0 for x in grads[:5])
    assert torch.equal(grads[5].cpu(), inp["dht"])
