"""The C-ABI library loads, exports every symbol include/gdr.h declares, and
rejects invalid arguments on the host before anything is enqueued (CPU only:
no call here reaches a kernel launch)."""
import ctypes
import math
import os
import re

import pytest
import torch

import gated_deltanet_chunked_rule_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = gdr.load_library()
    syms = header_symbols()
    assert "gdr_chunk_fwd" in syms and "gdr_chunk_bwd" in syms
    for s in syms:
        assert hasattr(lib, s), s


def shape(B=1, T=256, Hq=2, Hv=2, K=32, V=32, N=0, dtype=gdr.GDR_F32):
    return gdr._Shape(B, T, Hq, Hv, K, V, N, dtype)


def ws_size(sh, opts=None, cu=None):
    lib = gdr.load_library()
    cu_arr = None if cu is None else (ctypes.c_int32 * len(cu))(*cu)
    return lib.gdr_chunk_fwd_workspace_size(ctypes.byref(sh), None if opts is None else ctypes.byref(opts),
                                            cu_arr)


def last_error():
    return gdr.load_library().gdr_last_error().decode()


@pytest.mark.parametrize("kw,msg", [
    (dict(Hq=3, Hv=4), "multiple of Hq"),
    (dict(K=48, V=48), "K must be 32, 64 or 128"),
    (dict(K=64, V=32), "K must equal V"),
    (dict(K=128, V=128, dtype=gdr.GDR_F32), "fp32 supports K <= 64"),
    (dict(dtype=7), "dtype"),
    (dict(B=0), "positive"),
])
def test_workspace_size_rejects_bad_shapes(kw, msg):
    assert ws_size(shape(**kw)) == 0
    assert msg in last_error()


@pytest.mark.parametrize("cu,msg", [
    ([0, 10, 5, 256], "non-decreasing"),
    ([1, 100, 256], "cu_seqlens[0] must be 0"),
    ([0, 100, 200], "must equal T"),
])
def test_workspace_size_rejects_bad_cu_seqlens(cu, msg):
    assert ws_size(shape(N=len(cu) - 1), cu=cu) == 0
    assert msg in last_error()


def test_packed_mode_requires_B1():
    assert ws_size(shape(B=2, N=1), cu=[0, 256]) == 0
    assert "B == 1" in last_error()


def _fake(n):  # aligned, never dereferenced: validation fails first
    return ctypes.c_void_p(0x10000 * (n + 1))


def call_fwd(sh, scale=1.0, ws_bytes=1 << 40, opts=None, cu=None, cu_host=None, misalign=False):
    lib = gdr.load_library()
    p = [_fake(i) for i in range(12)]
    if misalign:
        p[0] = ctypes.c_void_p(0x10008)
    return lib.gdr_chunk_fwd(ctypes.byref(sh), opts, p[0], p[1], p[2], p[3], p[4], ctypes.c_float(scale),
                             None, cu, cu_host, p[5], None, None, None, p[6], ctypes.c_size_t(ws_bytes), None)


def test_fwd_rejects_before_launch():
    assert call_fwd(shape(Hq=3, Hv=4)) == -1
    assert call_fwd(shape(K=48, V=48)) == -2
    assert call_fwd(shape(), scale=float("nan")) == -1 and "scale" in last_error()
    assert call_fwd(shape(), scale=-1.0) == -1
    assert call_fwd(shape(), ws_bytes=16) == -3 and "workspace too small" in last_error()
    assert call_fwd(shape(), misalign=True) == -1 and "aligned" in last_error()
    cu_host = (ctypes.c_int32 * 2)(0, 256)
    assert call_fwd(shape(N=1), cu=None, cu_host=cu_host) == -1 and "without cu_seqlens" in last_error()
    assert call_fwd(shape(N=1), cu=_fake(20), cu_host=None) == -1 and "cu_seqlens_host" in last_error()


def test_bwd_rejects_before_launch():
    lib = gdr.load_library()
    p = [_fake(i) for i in range(20)]
    sh = shape(Hq=2, Hv=3)
    rc = lib.gdr_chunk_bwd(ctypes.byref(sh), None, *p[:5], None, p[5], None, ctypes.c_float(1.0), None,
                           None, None, *p[6:12], p[12], ctypes.c_size_t(1 << 40), None)
    assert rc == -1 and "multiple of Hq" in last_error()
    sh = shape()
    rc = lib.gdr_chunk_bwd(ctypes.byref(sh), None, *p[:5], None, p[5], None, ctypes.c_float(1.0), None,
                           None, None, *p[6:12], p[12], ctypes.c_size_t(8), None)
    assert rc == -3


def plan(B, T, Hq, Hv, K, cu=None, mode=gdr.CP_AUTO, seg=0, warm=0):
    q = torch.empty((B, T, Hq, K), dtype=torch.bfloat16, device="meta")
    v = torch.empty((B, T, Hv, K), dtype=torch.bfloat16, device="meta")
    return gdr.gdr_chunk_fwd_plan(q, v, cu, gdr.Options(mode, seg, warm))


def test_precise_vnew_option_is_validated():
    q = torch.empty((1, 256, 2, 128), dtype=torch.bfloat16, device="meta")
    v = torch.empty((1, 256, 4, 128), dtype=torch.bfloat16, device="meta")
    assert gdr.gdr_chunk_fwd_plan(q, v, None, gdr.Options(precise_vnew=1))["total_chunks"] == 4
    with pytest.raises(gdr.GdrError, match="precise_vnew"):
        gdr.gdr_chunk_fwd_plan(q, v, None, gdr.Options(precise_vnew=2))


def test_planner_cp_for_few_heads_long_context():
    info = plan(1, 65536, 4, 8, 128)
    assert info["total_chunks"] == 1024 and info["v_blocks"] == 1
    assert info["segment_chunks"] < 1024 and info["warmup_chunks"] == 8
    assert info["state_workgroups"] >= 256         # fills the 256 CUs


def test_planner_no_cp_when_units_fill_the_gpu():
    info = plan(1, 131072, 16, 64, 128, cu=torch.tensor([0, 65536, 131072], dtype=torch.int32))
    assert info["num_seqs"] == 2 and info["total_chunks"] == 2048
    info = plan(4, 8192, 32, 64, 128)
    assert info["segment_chunks"] == info["max_chunks"] and info["warmup_chunks"] == 0


def test_planner_forced_and_off():
    info = plan(1, 4096, 2, 2, 64, mode=gdr.CP_FORCE, seg=8, warm=3)
    assert info["segment_chunks"] == 8 and info["total_segments"] == 8 and info["warmup_chunks"] == 3
    info = plan(1, 65536, 4, 8, 128, mode=gdr.CP_OFF)
    assert info["segment_chunks"] == 1024 and info["total_segments"] == 1


def test_planner_ragged_and_empty_sequences():
    cu = torch.tensor([0, 0, 65, 65, 200], dtype=torch.int32)
    info = plan(1, 200, 1, 1, 32, cu=cu)
    assert info["num_seqs"] == 4
    assert info["total_chunks"] == 0 + 2 + 0 + 3 and info["max_chunks"] == 3
    assert info["total_segments"] == 4             # every sequence gets a state work item


def test_bwd_fp32_k64_unsupported():
    lib = gdr.load_library()
    sh = shape(K=64, V=64)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(sh), None, None) == 0
    assert "fp32 backward" in last_error()


def _bwd_args(B=1, T=130, Hq=2, Hv=4, K=64, N=None):
    """CPU tensors of matching shapes for gdr_chunk_bwd (never launched)."""
    N = B if N is None else N
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt)
    return dict(q=z(B, T, Hq, K), k=z(B, T, Hq, K), v=z(B, T, Hv, K), g=z(B, T, Hv, dt=torch.float32),
                beta=z(B, T, Hv, dt=torch.float32), A=z(B, T, Hv, 64, dt=torch.float32), do=z(B, T, Hv, K),
                dht=z(N, Hv, K, K, dt=torch.float32), initial_state=z(N, Hv, K, K, dt=torch.float32))


def _call_bwd(a, cu_seqlens=None):
    return gdr.gdr_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A"], a["do"], a["dht"], None,
                             a["initial_state"], cu_seqlens)


@pytest.mark.parametrize("name,bad", [
    ("k", (1, 130, 2, 32)), ("k", (1, 130, 1, 64)), ("v", (1, 129, 4, 64)), ("g", (1, 130, 2)),
    ("beta", (1, 130, 4, 1)), ("A", (1, 130, 4, 32)), ("do", (1, 130, 4, 32)), ("dht", (2, 4, 64, 64)),
    ("initial_state", (1, 4, 64, 32)),
])
def test_bwd_binding_rejects_mismatched_shapes(name, bad):
    # Every tensor's shape is checked against q and v before anything reaches
    # the library (whose C ABI sees bare pointers); CPU tensors show the order:
    # a shape error comes first, and matching shapes only then fail on the
    # device check, so no call here gets near a launch.
    a = _bwd_args()
    a[name] = torch.zeros(bad, dtype=a[name].dtype)
    with pytest.raises(gdr.GdrError, match=f"shape mismatch: {name} "):
        _call_bwd(a)


def test_bwd_binding_checks_states_against_packed_sequences():
    a = _bwd_args(T=200, N=3)
    cu = torch.tensor([0, 70, 70, 200], dtype=torch.int32)
    with pytest.raises(gdr.GdrError, match="must be a device tensor"):
        _call_bwd(a, cu)                    # N = 3 sequences: states [3, Hv, K, V] match
    a["dht"] = torch.zeros((1, 4, 64, 64))
    with pytest.raises(gdr.GdrError, match="shape mismatch: dht "):
        _call_bwd(a, cu)


def test_fwd_binding_rejects_mismatched_shapes():
    a = _bwd_args()
    with pytest.raises(gdr.GdrError, match="must be a device tensor"):
        gdr.gdr_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], None, a["initial_state"])
    with pytest.raises(gdr.GdrError, match="shape mismatch: beta "):
        gdr.gdr_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"][:, :5], None, a["initial_state"])
    with pytest.raises(gdr.GdrError, match="shape mismatch: initial_state "):
        gdr.gdr_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], None, a["initial_state"][:, :2])


def test_noalloc_rejects_problems_beyond_the_scratch():
    # The packed workload shape (131072 tokens, Hv = 64) needs about 1.1 GiB
    # of workspace, beyond the no-allocation entry point's 128 MiB scratch:
    # rejected on the host, before the scratch is looked up or anything is
    # enqueued (fake, never dereferenced pointers).
    lib = gdr.load_library()
    sh = shape(B=1, T=131072, Hq=16, Hv=64, K=128, V=128, dtype=gdr.GDR_BF16)
    p = [_fake(i) for i in range(8)]
    rc = lib.gdr_chunk_fwd_noalloc(ctypes.byref(sh), None, p[0], p[1], p[2], p[3], p[4], ctypes.c_float(1.0),
                                   None, None, None, p[5], None, None, None, None)
    assert rc == -3 and "beyond the library scratch" in last_error()
    sh = shape(B=1, T=65536, Hq=4, Hv=8, K=128, V=128, dtype=gdr.GDR_BF16)
    assert ws_size(sh) <= (128 << 20)    # the long-context shape fits


def test_peak_probe_library_exports_its_header():
    # the measured-peak probes (copy kernel, MFMA loops) live in their own
    # library; every function its header declares is exported, and invalid
    # arguments are refused on the host
    path = os.path.join(ROOT, "gated_deltanet_chunked_rule_amd", "libgdr_peaks.so")
    lib = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gdr_peaks.h")).read(), flags=re.S)
    syms = sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))
    assert syms == ["gdr_peak_copy", "gdr_peak_mfma_bf16"]
    for s in syms:
        assert hasattr(lib, s), s
    ms = ctypes.c_float()
    lib.gdr_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    assert lib.gdr_peak_copy(_fake(1), _fake(2), 100, 1, None, ctypes.byref(ms)) == -1   # not a multiple of 16
    lib.gdr_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    assert lib.gdr_peak_mfma_bf16(_fake(1), 8, 10, 1, 1, None, ctypes.byref(ms)) == -1  # tile 8 does not exist
