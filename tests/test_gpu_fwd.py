"""Forward parity of the HIP path (through the C ABI) against the fp64 oracle.

Metric: err(x) = max|x - ref| / max|ref| per output; bf16 workloads must reach
2e-2 on o and 1e-2 on final_state, fp32 workloads 1e-4."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_rule_amd as gdr
import gdr_inputs as gi
import oracle
from parity import TOL, dev, f64, gpu_fwd, head_mass_inputs, oracle_fwd, rel_err, set_chunk_gate_mass

pytestmark = pytest.mark.gpu


def check_fwd(inp, options=None, heads=None, t_max=0, label=""):
    w = inp["workload"]
    print(f"[fwd] {label or w.name} B={w.B} T={inp['q'].shape[1]} Hq={w.Hq} Hv={w.Hv} K={w.K} "
          f"{w.dtype} opts={options}", flush=True)
    o, ht, _, _ = gpu_fwd(inp, options)
    torch.cuda.synchronize()
    ro, rht = oracle_fwd(inp, heads=heads, t_max=t_max)
    tol = TOL[w.dtype]
    eo, eh = rel_err(o, ro), rel_err(ht, rht) if not t_max else 0.0
    print(f"      err(o)={eo:.3e} err(final_state)={eh:.3e}", flush=True)
    assert np.isfinite(eo) and eo <= tol["o"], eo
    assert np.isfinite(eh) and eh <= tol["final_state"], eh
    return o, ht


def test_tiny_fp32_workload():
    check_fwd(gi.make_inputs(gi.WORKLOADS["tiny_fp32"]))


@pytest.mark.parametrize("dtype,K", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 32), ("f32", 64)])
def test_ragged_tail_with_initial_state(dtype, K):
    w = gi.custom(B=2, T=64 * 3 + 17, Hq=2, Hv=4, K=K, V=K, dtype=dtype, seed=21, initial_state=True)
    check_fwd(gi.make_inputs(w))


@pytest.mark.parametrize("G,K", [(1, 64), (2, 64), (4, 64), (8, 64), (8, 128)])
def test_grouped_heads(G, K):
    w = gi.custom(B=1, T=300, Hq=2, Hv=2 * G, K=K, V=K, dtype="bf16", seed=22 + G + K)
    check_fwd(gi.make_inputs(w))


def test_varlen_with_empty_and_ragged_sequences():
    w = gi.custom(B=1, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=30, initial_state=True)
    inp = gi.packed_from_lengths(w, [1, 63, 64, 0, 65, 200, 130])
    check_fwd(inp)


def test_varlen_equals_separate_calls():
    w = gi.custom(B=1, Hq=2, Hv=4, K=64, V=64, dtype="bf16", seed=31, initial_state=True)
    lens = [70, 129, 64]
    inp = gi.packed_from_lengths(w, lens)
    o, ht, _, _ = gpu_fwd(inp)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        one = dict(inp, q=inp["q"][:, s:e], k=inp["k"][:, s:e], v=inp["v"][:, s:e], g=inp["g"][:, s:e],
                   beta=inp["beta"][:, s:e], initial_state=inp["initial_state"][n:n + 1], cu_seqlens=None)
        o1, h1, _, _ = gpu_fwd(one)
        assert torch.equal(o1, o[:, s:e]) and torch.equal(h1[0], ht[n])


def test_state_continuation_split_equals_one_call():
    w = gi.custom(B=1, T=1000, Hq=1, Hv=2, K=128, V=128, dtype="bf16", seed=32, initial_state=True)
    inp = gi.make_inputs(w)
    o, ht, _, _ = gpu_fwd(inp)
    cut = 437
    a = {k: (v[:, :cut] if k in ("q", "k", "v", "g", "beta") else v) for k, v in inp.items()}
    oa, ha, _, _ = gpu_fwd(a)
    b = {k: (v[:, cut:] if k in ("q", "k", "v", "g", "beta") else v) for k, v in inp.items()}
    b["initial_state"] = ha.cpu()
    ob, hb, _, _ = gpu_fwd(b)
    ro, rht = oracle_fwd(inp)
    assert rel_err(torch.cat([oa, ob], 1), ro) <= TOL["bf16"]["o"]
    assert rel_err(hb, rht) <= TOL["bf16"]["final_state"]
    assert rel_err(torch.cat([oa, ob], 1), f64(o)) <= TOL["bf16"]["o"]


@pytest.mark.parametrize("seg,warm", [(4, 2), (8, 8), (3, 1)])
def test_context_parallel_split_matches_oracle(seg, warm):
    # decaying gates: every warmup window is certified; results equal the
    # serial ones up to exp(sum g) * |S| and different rounding.
    w = gi.custom(B=1, T=64 * 37 + 5, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=40, initial_state=True,
                  gate=(0.5, 0.9))
    inp = gi.make_inputs(w)
    ocp, hcp = check_fwd(inp, gdr.Options(gdr.CP_FORCE, seg, warm), label=f"cp seg={seg} warm={warm}")
    ooff, hoff, _, _ = gpu_fwd(inp, gdr.Options(gdr.CP_OFF))
    assert rel_err(ocp, f64(ooff)) <= TOL["bf16"]["o"]


@pytest.mark.parametrize("dtype,K,cp", [("bf16", 128, False), ("bf16", 128, True), ("f32", 32, False)])
def test_strong_decay_gates(dtype, K, cp):
    # gates alpha = e^g in (1e-6, 1e-2): the in-chunk decay e^gamma underflows
    # fp32 within a chunk (gamma reaches several hundred below zero), so every
    # factor of the chunk form must come from differences of gamma; the state
    # forgets within a few tokens and o is dominated by the intra-chunk terms
    w = gi.custom(B=2, T=64 * 5 + 13, Hq=2, Hv=4, K=K, V=K, dtype=dtype, seed=46, initial_state=True,
                  gate=(1e-6, 1e-2))
    inp = gi.make_inputs(w)
    check_fwd(inp, gdr.Options(gdr.CP_FORCE, 2, 1) if cp else None, label=f"strong decay cp={cp}")


def test_context_parallel_uncertified_heads_fall_back():
    # g == 0 on some heads: warmup from zero is not accurate there, so those
    # heads must be computed serially and still match the oracle.
    w = gi.custom(B=1, T=64 * 40, Hq=4, Hv=8, K=128, V=128, dtype="bf16", seed=41, initial_state=True,
                  gate=(0.9, 0.999), zero_gate_frac=0.3)
    inp = gi.make_inputs(w)
    check_fwd(inp, gdr.Options(gdr.CP_FORCE, 5, 2), label="cp with g=0 heads")


def test_auxiliary_outputs_g_cum_and_A():
    w = gi.custom(B=1, Hq=2, Hv=4, K=64, V=64, dtype="bf16", seed=50)
    inp = gi.packed_from_lengths(w, [100, 64, 33])
    _, _, gc, A = gpu_fwd(inp, output_g_cum=True, output_A=True)
    cu = inp["cu_seqlens"].numpy()
    rg = oracle.chunk_gcum(f64(inp["g"]), cu)
    rA = oracle.chunk_A(f64(inp["k"]), f64(inp["g"]), f64(inp["beta"]), 4, cu)
    eg, eA = float(np.max(np.abs(f64(gc) - rg))), rel_err(A, rA)
    print(f"[fwd] g_cum max abs err {eg:.3e}, A err {eA:.3e}", flush=True)
    # fp32 outputs of bf16 inputs: exact up to fp32 rounding (K K^T of bf16
    # keys is exact in fp32 products; the cumsum, the decays and the blocked
    # inverse add a few ulps), so a half-precision A would fail by far
    assert eg <= 1e-5
    assert eA <= 1e-5


def test_deterministic():
    w = gi.custom(B=1, T=64 * 20 + 3, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=60, initial_state=True)
    inp = gi.make_inputs(w)
    o1, h1, _, _ = gpu_fwd(inp)
    o2, h2, _, _ = gpu_fwd(inp)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_edge_prefill_workload_full_size():
    check_fwd(gi.make_inputs(gi.WORKLOADS["edge_prefill"]))


def test_long_context_workload_full_size():
    # the benchmarked configuration, with the automatic CP split
    inp = gi.make_inputs(gi.WORKLOADS["long_context"])
    info = gdr.gdr_chunk_fwd_plan(inp["q"], inp["v"])
    assert info["warmup_chunks"] > 0
    check_fwd(inp)


def test_one_head_quarter_million_tokens():
    # one value head over 262144 tokens (4096 chunks): the automatic split
    # gives the single head 256 segments, each with its own warmup window
    w = gi.custom(B=1, T=262144, Hq=1, Hv=1, K=128, V=128, dtype="bf16", seed=47, initial_state=True)
    inp = gi.make_inputs(w)
    info = gdr.gdr_chunk_fwd_plan(inp["q"], inp["v"])
    print(f"      plan: {info}", flush=True)
    assert info["total_segments"] >= 128 and info["warmup_chunks"] > 0
    check_fwd(inp, label="one head, 262144 tokens")


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f32", 64)])
def test_odd_head_counts_and_many_short_rows(dtype, K):
    # three q/k heads (six value heads) and 48 rows of 70 tokens: head and row
    # counts that are not multiples of the XCD count or of two
    w = gi.custom(B=48, T=70, Hq=3, Hv=6, K=K, V=K, dtype=dtype, seed=49, initial_state=True)
    check_fwd(gi.make_inputs(w), label="Hq=3 Hv=6 B=48")


def test_varlen_workload_full_size_all_heads():
    # Every value head of the packed workload (16 sequences, 131072 tokens,
    # Hv = 64) against the oracle, o and final_state element by element.  The
    # oracle runs one q/k head group at a time (4 q/k heads = 16 value heads,
    # sliced consistently with the head map) to bound host memory.
    inp = gi.make_inputs(gi.WORKLOADS["varlen"])
    w = inp["workload"]
    G = w.Hv // w.Hq
    print(f"[fwd] varlen lengths={np.diff(inp['cu_seqlens'].numpy()).tolist()}", flush=True)
    o, ht, _, _ = gpu_fwd(inp)
    torch.cuda.synchronize()
    o, ht = o.cpu(), ht.cpu()
    worst_o = worst_h = 0.0
    for a in range(0, w.Hq, 4):
        b = min(w.Hq, a + 4)
        part = dict(inp, q=inp["q"][:, :, a:b], k=inp["k"][:, :, a:b], v=inp["v"][:, :, a * G:b * G],
                    g=inp["g"][:, :, a * G:b * G], beta=inp["beta"][:, :, a * G:b * G],
                    initial_state=inp["initial_state"][:, a * G:b * G])
        ro, rht = oracle_fwd(part)
        eo, eh = rel_err(o[:, :, a * G:b * G], ro), rel_err(ht[:, a * G:b * G], rht)
        print(f"      value heads [{a * G},{b * G}) err(o)={eo:.3e} err(final_state)={eh:.3e}", flush=True)
        assert eo <= TOL["bf16"]["o"] and eh <= TOL["bf16"]["final_state"], (a, eo, eh)
        worst_o, worst_h = max(worst_o, eo), max(worst_h, eh)
    print(f"      all 64 value heads: worst err(o)={worst_o:.3e} err(final_state)={worst_h:.3e}", flush=True)


def test_context_parallel_warmup_is_really_used():
    # Weakly decaying heads: one warmup chunk leaves a large error.  With the
    # default certificate those heads run serially (exact); with the threshold
    # loosened past their gate mass they take the warmup path and the outputs
    # visibly deviate -- so the segmented path is the one normally running and
    # the certificate is what keeps uncertifiable heads exact.
    w = gi.custom(B=1, T=64 * 24, Hq=1, Hv=2, K=128, V=128, dtype="bf16", seed=42, initial_state=True,
                  gate=(0.999, 1.0))
    inp = gi.make_inputs(w)
    ro, _ = oracle_fwd(inp)
    o_ok, _, _, _ = gpu_fwd(inp, gdr.Options(gdr.CP_FORCE, 4, 1))
    assert rel_err(o_ok, ro) <= TOL["bf16"]["o"]
    o_bad, _, _, _ = gpu_fwd(inp, gdr.Options(gdr.CP_FORCE, 4, 1, -1e-4))
    assert rel_err(o_bad, ro) > 5e-2


# Per-chunk gate masses repeating (-0.5, -20, -1): the chunk just before each
# segment start (and the first after each segment end) decays weakly, the one
# beyond it strongly, so every segment needs a warmup of exactly two chunks
# to meet ln(1e-6).  A one-chunk warmup leaves an error of e^-1 (forward) or
# e^-0.5 (reverse) times the state: the loosened run shows that size.
STEPPED_MASS = (-0.5, -20.0, -1.0)


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f32", 64)])
def test_short_warmup_takes_enough_chunks(dtype, K):
    w = gi.custom(B=1, T=64 * 12 + 5, Hq=1, Hv=2, K=K, V=K, dtype=dtype, seed=43, initial_state=True)
    inp = set_chunk_gate_mass(gi.make_inputs(w), lambda c: STEPPED_MASS[c % 3])
    check_fwd(inp, gdr.Options(gdr.CP_FORCE, 3, 4), label="stepped gates, warmup <= 4")
    ro, _ = oracle_fwd(inp)
    o_one, _, _, _ = gpu_fwd(inp, gdr.Options(gdr.CP_FORCE, 3, 1, -0.1))
    torch.cuda.synchronize()
    assert rel_err(o_one, ro) > 5e-2


def test_short_warmup_longer_than_a_wave():
    # Segment 1 starts at chunk 80, with up to 100 warmup chunks allowed.  In
    # chunks 16..79 beta = 0 (the state only decays) with a gate mass of -0.02
    # per chunk, and chunk 15 carries -13: the shortest window that meets
    # ln(1e-6) is 65 chunks (-14.28), which spans two 64-lane blocks of the
    # window scan; 64 chunks would leave e^-1.28 of the state.  The control
    # certifies a 50-chunk window (mass -1) and must miss.
    w = gi.custom(B=1, T=64 * 160, Hq=1, Hv=1, K=64, V=64, dtype="bf16", seed=45, initial_state=True)
    inp = set_chunk_gate_mass(gi.make_inputs(w), lambda c: -0.02 if 16 <= c < 80 else (-13.0 if c == 15 else -1.0))
    beta = inp["beta"].clone()
    beta[:, 16 * 64:80 * 64, :] = 0.0
    inp["beta"] = beta
    check_fwd(inp, gdr.Options(gdr.CP_FORCE, 80, 100), label="65-chunk warmup")
    ro, _ = oracle_fwd(inp)
    o_short, _, _, _ = gpu_fwd(inp, gdr.Options(gdr.CP_FORCE, 80, 64, -1.0))
    torch.cuda.synchronize()
    assert rel_err(o_short, ro) > 5e-2


def test_warmup_length_differs_per_head_varlen():
    check_fwd(head_mass_inputs(), gdr.Options(gdr.CP_FORCE, 3, 8), label="per-head warmups, varlen, G=4")


@pytest.mark.parametrize("dtype,K,spread", [("bf16", 128, 0.3), ("bf16", 128, 0.15), ("f32", 64, 0.05)])
def test_nearly_parallel_keys_without_decay(dtype, K, spread):
    # Strongly coupled intra-chunk systems (I + L): keys share one direction
    # (spread = size of the per-token deviation), beta = 1, g = 0, so L is
    # close to the all-ones lower triangle.  fp32 is checked at the extreme;
    # bf16 down to spread 0.15 (err(o) about 0.016): with closer keys and no
    # decay the bf16 roundings of A diag(beta), P and Vnew (the MFMA operands
    # of the chunk products) exceed the bf16 tolerance (0.021 at spread 0.1,
    # 0.06 at 0.05), whatever the inverse.
    w = gi.custom(B=1, T=64 * 5 + 9, Hq=2, Hv=4, K=K, V=K, dtype=dtype, seed=70)
    inp = gi.make_inputs(w)
    gen = torch.Generator().manual_seed(70)
    T = inp["k"].shape[1]
    k = torch.randn(1, 1, 2, K, generator=gen) + spread * torch.randn(1, T, 2, K, generator=gen)
    inp["k"] = (k / k.norm(dim=-1, keepdim=True)).to(inp["k"].dtype)
    inp["beta"] = torch.ones_like(inp["beta"])
    inp["g"] = torch.zeros_like(inp["g"])
    check_fwd(inp, label=f"nearly parallel keys {dtype}")


def test_nearly_parallel_keys_precise_vnew():
    # The same coupled system at spread 0.1, where the single bf16 roundings
    # of the chunk products' operands reach err(o) of about 0.021: with
    # precise_vnew the output pass takes Vnew as two bf16 terms in P Vnew and
    # in the state update (an fp64 emulation of the rounded chunk path puts
    # err(o) at 0.0167 with Vnew exact and everything else rounded).
    K, spread = 128, 0.1
    w = gi.custom(B=1, T=64 * 5 + 9, Hq=2, Hv=4, K=K, V=K, dtype="bf16", seed=70)
    inp = gi.make_inputs(w)
    gen = torch.Generator().manual_seed(70)
    T = inp["k"].shape[1]
    k = torch.randn(1, 1, 2, K, generator=gen) + spread * torch.randn(1, T, 2, K, generator=gen)
    inp["k"] = (k / k.norm(dim=-1, keepdim=True)).to(inp["k"].dtype)
    inp["beta"] = torch.ones_like(inp["beta"])
    inp["g"] = torch.zeros_like(inp["g"])
    ro, _ = oracle_fwd(inp)
    o1, _, _, _ = gpu_fwd(inp)
    print(f"      one bf16 term: err(o)={rel_err(o1, ro):.3e}", flush=True)
    o2, _ = check_fwd(inp, gdr.Options(precise_vnew=1), label="nearly parallel keys, precise Vnew")
    assert rel_err(o2, ro) < rel_err(o1, ro)


@pytest.mark.parametrize("dtype,K,seg", [("bf16", 128, 3), ("bf16", 64, 1), ("f32", 32, 2)])
def test_exact_segments_for_uncertified_heads(dtype, K, seg):
    # g = 0 on every head: no warmup window is certified, so every head takes
    # the exact path (segment transitions, scan, then the segments from their
    # exact start states), here with an initial state and a ragged tail.
    w = gi.custom(B=2, T=64 * 11 + 23, Hq=2, Hv=4, K=K, V=K, dtype=dtype, seed=80, initial_state=True,
                  zero_gate_frac=1.0)
    check_fwd(gi.make_inputs(w), gdr.Options(gdr.CP_FORCE, seg, 2), label=f"exact segments L={seg}")


def test_serial_fallback_option_for_uncertified_heads():
    w = gi.custom(B=1, T=64 * 24 + 5, Hq=2, Hv=8, K=128, V=128, dtype="bf16", seed=81, initial_state=True,
                  gate=(0.9, 0.999), zero_gate_frac=0.5)
    inp = gi.make_inputs(w)
    o1, h1 = check_fwd(inp, gdr.Options(gdr.CP_FORCE, 4, 2, 0.0, 1), label="serial fallback")
    o2, h2 = check_fwd(inp, gdr.Options(gdr.CP_FORCE, 4, 2, 0.0, 0), label="exact segments")
    # both reach the same recurrence; they differ only by rounding order
    assert rel_err(o1, f64(o2)) <= 2e-2 and rel_err(h1, f64(h2)) <= 1e-2


def test_exact_segments_varlen():
    w = gi.custom(B=1, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=82, initial_state=True,
                  gate=(0.9, 0.999), zero_gate_frac=0.5)
    inp = gi.packed_from_lengths(w, [64 * 9 + 7, 1, 64 * 3, 0, 64 * 6 + 40])
    check_fwd(inp, gdr.Options(gdr.CP_FORCE, 2, 1), label="varlen exact segments")


def test_workspace_filled_with_nan():
    # the forward writes every workspace element it reads (the A diag(beta)
    # rows with their zero blocks, the gate cumsums, the certificates): a
    # workspace of NaN bit patterns changes nothing; the returned A is zero
    # above each chunk's diagonal
    w = gi.custom(B=1, T=64 * 3 + 8, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=77, initial_state=True)
    inp = gi.make_inputs(w)
    nbytes = gdr.fwd_workspace_bytes(dev(inp["q"]), dev(inp["v"]))
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    print(f"[fwd] NaN-filled workspace T={w.T}", flush=True)
    o, ht, _, A = gpu_fwd(inp, output_A=True, workspace=ws)
    torch.cuda.synchronize()
    ro, rht = oracle_fwd(inp)
    assert rel_err(o, ro) <= TOL["bf16"]["o"] and rel_err(ht, rht) <= TOL["bf16"]["final_state"]
    a = f64(A)   # [B, T, Hv, 64]: row t of its chunk's A
    pos = np.arange(w.T) % 64
    upper = np.arange(64)[None, :] > pos[:, None]
    assert np.isfinite(a).all() and np.all(a[0][upper[:, None, :].repeat(w.Hv, 1)] == 0.0)


def test_graph_replay_matches_eager():
    # The forward enqueues kernels only (no allocation, memset or sync inside
    # the library), so one call can be captured in a HIP graph and replayed;
    # every replay, with eager work in between, equals the eager call bitwise.
    w = gi.custom(B=1, T=64 * 40 + 5, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=78, initial_state=True)
    inp = gi.make_inputs(w)
    q, k, v, g, b, h0 = (dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "initial_state"))
    opts = gdr.Options(gdr.CP_FORCE, 8, 2)   # CP segments: transition, scan and output launches
    print(f"[fwd] graph replay T={w.T}", flush=True)
    call = lambda: gdr.gdr_chunk_fwd(q, k, v, g, b, inp["scale"], h0, options=opts)
    o_ref, ht_ref, _, _ = call()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, ht_g, _, _ = call()
    for i in range(3):
        o_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(ht_g, ht_ref), i
        o_e, _, _, _ = call()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_ref)


@pytest.mark.parametrize("T", [0, 1, 64])
def test_empty_single_token_and_one_chunk(T):
    # T = 0: no chunk at all, the final state is the initial state; T = 1: a
    # one-token chunk; T = 64: exactly one full chunk
    w = gi.custom(B=2, T=T, Hq=2, Hv=4, K=128, V=128, dtype="bf16", seed=79, initial_state=True)
    inp = gi.make_inputs(w)
    print(f"[fwd] T={T}", flush=True)
    o, ht, _, _ = gpu_fwd(inp)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (2, T, 4, 128)
    if T == 0:
        assert torch.equal(ht.cpu(), inp["initial_state"])
        return
    ro, rht = oracle_fwd(inp)
    assert rel_err(o, ro) <= TOL["bf16"]["o"] and rel_err(ht, rht) <= TOL["bf16"]["final_state"]


def test_zero_beta_state_only_decays():
    # beta = 0 writes nothing: S_t = exp(g_1 + .. + g_t) S_0, so the closed form
    # o_t = scale exp(sum_{u<=t} g_u) S_0^T q_t and final S = exp(sum g) S_0 fix
    # the outputs without the oracle (fp32: bf16 q, k, v are exact inputs here)
    w = gi.custom(B=1, T=64 * 3 + 10, Hq=2, Hv=4, K=64, V=64, dtype="f32", seed=80, initial_state=True)
    inp = gi.make_inputs(w)
    inp["beta"] = torch.zeros_like(inp["beta"])
    print(f"[fwd] beta = 0, T={w.T}", flush=True)
    o, ht, _, _ = gpu_fwd(inp)
    torch.cuda.synchronize()
    q, g, s0 = f64(inp["q"])[0], f64(inp["g"])[0], f64(inp["initial_state"])[0]   # [T,Hq,K], [T,Hv], [Hv,K,V]
    G = w.Hv // w.Hq
    decay = np.exp(np.cumsum(g, axis=0))                                          # [T, Hv]
    qv = np.repeat(q, G, axis=1)                                                  # [T, Hv, K]
    ro = inp["scale"] * decay[:, :, None] * np.einsum("thk,hkv->thv", qv, s0)
    rht = decay[-1][:, None, None] * s0
    assert rel_err(o[0], ro) <= TOL["f32"]["o"]
    assert rel_err(ht[0], rht) <= TOL["f32"]["final_state"]


def test_certificate_excludes_positive_gates_and_expanding_keys():
    # Every head decays fast (gate mass -7.5 per chunk: a 2-chunk warmup meets
    # ln(1e-6)), so by its windows alone every head would take the warmup
    # path.  Head 1 has three tokens with g > 0 and head 2 one token with
    # beta |k|^2 = 3 (a transition that expands the state), both in chunks
    # that lie in no warmup window (segments of 6 chunks, windows of 2: chunks
    # 4-5 and 10-11).  Such heads must not be certified: a warmup error could
    # grow there.  With the serial fallback an uncertified head runs whole,
    # so its outputs equal the unsegmented call bitwise, while a certified
    # head's outputs at a segment start carry the warmup's e^-15 relative
    # error and differ in fp32.  The default (exact segment states) matches
    # the oracle on every head.
    w = gi.custom(B=1, T=64 * 16 + 9, Hq=4, Hv=4, K=64, V=64, dtype="f32", seed=47, initial_state=True)
    inp = set_chunk_gate_mass(gi.make_inputs(w), lambda c: -7.5)
    g, beta = inp["g"].clone(), inp["beta"].clone()
    g[0, 8 * 64 + 10:8 * 64 + 13, 1] = 0.2
    beta[0, 9 * 64 + 20, 2] = 3.0
    inp["g"], inp["beta"] = g, beta
    check_fwd(inp, gdr.Options(gdr.CP_FORCE, 6, 2), label="g > 0 and beta |k|^2 > 2 in segment bodies")
    o_off, h_off, _, _ = gpu_fwd(inp, gdr.Options(gdr.CP_OFF))
    o_ser, h_ser, _, _ = gpu_fwd(inp, gdr.Options(gdr.CP_FORCE, 6, 2, 0.0, 1))
    torch.cuda.synchronize()
    for h in (1, 2):
        assert torch.equal(o_ser[:, :, h], o_off[:, :, h]) and torch.equal(h_ser[:, h], h_off[:, h]), h
    seg1 = slice(6 * 64, 7 * 64)   # first chunk of segment 1
    for h in (0, 3):
        assert not torch.equal(o_ser[:, seg1, h], o_off[:, seg1, h]), h
