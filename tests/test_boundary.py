"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/fa2.h declares, and rejects bad arguments before any HIP
call (so no compute call is made here)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import exact_attention_fwd_amd as fa2
from exact_attention_fwd_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa2.LIB_PATH):
        _build.build()
    return fa2.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa[12]_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(fa2.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_probe_library_rejects_bad_arguments_before_any_hip_call():
    # the measurement aids behind bench.py --lds-probe / --valu-probe / --step-probe, a library of their own
    if not os.path.exists(_build.PROBE_PATH):
        _build.build_probe()
    probe = ctypes.CDLL(_build.PROBE_PATH)
    f = probe.fa2probe_lds_read
    f.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_double)]
    f.restype = ctypes.c_int
    out = (ctypes.c_double * 3)()
    assert f(2, 256, 1, 1, 1, out) == 1       # no such mode
    assert f(0, 100, 1, 1, 1, out) == 1       # threads not whole waves
    assert f(1, 2048, 1, 1, 1, out) == 1      # more than 1024 threads
    assert f(0, 256, 0, 1, 1, out) == 1       # no workgroups
    assert f(0, 256, 1, 1, 1, None) == 1      # no output
    g = probe.fa2probe_valu_issue
    g.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_double)]
    g.restype = ctypes.c_int
    assert g(5, 256, 1, 1, out) == 1          # no such instruction kind
    assert g(0, 96, 1, 1, out) == 1           # threads not whole waves
    assert g(0, 256, 1, 0, out) == 1          # no iterations
    h = probe.fa2probe_step_model
    h.argtypes = [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_double)]
    h.restype = ctypes.c_int
    out4 = (ctypes.c_double * 4)()
    assert h(96, 0, 1, 1, 1, 2, 1, out4) == 1    # no model at this head dim
    assert h(64, 8, 1, 1, 1, 2, 1, out4) == 1    # no such mode
    assert h(64, 6, 1, 1, 1, 2, 1, out4) == 1    # the staging variants: two waves per SIMD only
    assert h(128, 7, 3, 1, 1, 2, 1, out4) == 1
    assert h(64, 2, 4, 1, 1, 2, 1, out4) == 1    # four waves per SIMD do not fit the pipelined step
    assert h(64, 3, 3, 1, 1, 2, 1, out4) == 1    # nor three with LDS operands
    assert h(64, 5, 4, 1, 1, 2, 1, out4) == 1    # the sequential step with LDS operands: at most three
    assert h(128, 2, 3, 1, 1, 2, 1, out4) == 1   # d = 128 pipelined: at most two
    assert h(128, 0, 4, 1, 1, 2, 1, out4) == 1   # d = 128 MFMAs alone: at most three
    assert h(128, 4, 1, 1, 1, 2, 1, out4) == 1   # d = 128 with barriers: two only
    assert h(64, 0, 1, 2, 1, 2, 1, out4) == 1    # operand data: 0 or 1
    assert h(64, 0, 0, 1, 1, 2, 1, out4) == 1    # no waves
    assert h(64, 0, 1, 1, 1, 3, 1, out4) == 1    # odd tile count
    assert h(64, 0, 1, 1, 0, 2, 1, out4) == 1    # no workgroups
    assert h(64, 0, 1, 1, 1, 2, 1, None) == 1    # no output


def test_version_and_status_strings(lib):
    assert fa2.fa2_version().startswith("fa2-gfx950")
    seen = set()
    for st in range(7):
        s = fa2.fa2_status_string(st)
        assert s and s not in seen
        seen.add(s)
    assert fa2.fa2_status_string(99) == "unknown status"
    assert fa2.fa2_last_hip_error() == 0


# Fake, 16-byte aligned, non-overlapping "device" addresses: every call below
# fails validation, which runs before the first HIP call.
Q, K, V, O, L = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20
GOOD = dict(B=1, H=1, N=16, d=64, scale=0.125, causal=0)


def call(q=Q, k=K, v=V, o=O, lse=L, **kw):
    a = dict(GOOD, **kw)
    return fa2.fa2_fwd(q, k, v, o, lse, a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], 0)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_null_pointer(lib, which):
    assert call(**{which: 0}) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value", [("B", 0), ("H", 0), ("N", 0), ("B", -1), ("N", (1 << 22) + 1)])
def test_bad_sizes(lib, field, value):
    assert call(**{field: value}) == fa2.FA2_ERR_INVALID_ARG


def test_too_many_rows(lib):
    assert call(B=1024, H=1024, N=4096) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_non_finite_scale(lib, scale):
    assert call(scale=scale) == fa2.FA2_ERR_INVALID_ARG


def _scale_limit(d):
    """Largest |scale| whose scaled scores of fp16 inputs all stay finite in
    fp32: |scale| * log2(e) * 65504^2 * d <= FLT_MAX."""
    return float(np.finfo(np.float32).max) / (math.log2(math.e) * 65504.0 ** 2 * d)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("sign", [1, -1])
def test_scale_beyond_the_fp32_score_range(lib, d, sign):
    lim = _scale_limit(d)
    below = float(np.float32(lim * (1 - 2 ** -20)))
    above = float(np.float32(lim * (1 + 2 ** -20)))
    # a misaligned Q, checked after the scale rule, shows that the largest
    # accepted scale passes it without reaching a HIP call
    assert call(q=Q + 2, d=d, scale=sign * below) == fa2.FA2_ERR_MISALIGNED
    assert call(d=d, scale=sign * above) == fa2.FA2_ERR_INVALID_ARG
    assert call(d=d, scale=sign * 1e37) == fa2.FA2_ERR_INVALID_ARG
    if d <= 128:
        assert bcall(d=d, scale=sign * above) == fa2.FA2_ERR_INVALID_ARG
        assert bcall(q=Q + 2, d=d, scale=sign * below) == fa2.FA2_ERR_MISALIGNED
        assert scall(d=d, scale=sign * above) == fa2.FA2_ERR_INVALID_ARG
        assert ncall(d=d, scale=sign * above) == fa2.FA2_ERR_INVALID_ARG
        assert ncall(k=K + 8, d=d, scale=sign * below) == fa2.FA2_ERR_MISALIGNED
    if d == 64:
        assert fcall(scale=sign * above) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [0, 16, 48, 63, 80, 160, 192, 512])
def test_unsupported_head_dim(lib, d):
    assert call(d=d) == fa2.FA2_ERR_UNSUPPORTED


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_sequence_length_limit_per_head_dim(lib, d):
    # N * d * 2 bytes per head must fit the 32-bit buffer offsets: N * d <=
    # 2^29 (and N <= 2^22).  A misaligned Q, checked after the length rule,
    # shows which lengths pass it without reaching a HIP call.
    n_max = min(1 << 22, (1 << 29) // d)
    assert call(q=Q + 2, N=n_max, d=d) == fa2.FA2_ERR_MISALIGNED
    assert call(q=Q + 2, N=n_max + 1, d=d) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_misaligned(lib, which):
    base = dict(q=Q, k=K, v=V, o=O, lse=L)
    assert call(**{which: base[which] + 8}) == fa2.FA2_ERR_MISALIGNED


def test_overlapping_outputs(lib):
    assert call(o=Q) == fa2.FA2_ERR_INVALID_ARG
    assert call(o=K + 1024) == fa2.FA2_ERR_INVALID_ARG          # inside k's 2 KiB
    assert call(lse=V + 16) == fa2.FA2_ERR_INVALID_ARG
    assert call(lse=O + 2032) == fa2.FA2_ERR_INVALID_ARG        # inside o


def test_python_wrapper_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa2.fwd(x, x, x)


def test_missing_library_fails_loudly(tmp_path):
    from exact_attention_fwd_amd import _lib
    saved = _lib._lib
    try:
        _lib._lib = None
        with pytest.raises(RuntimeError, match="no non-HIP fallback"):
            _lib.load_library(str(tmp_path / "libfa2.so"))
    finally:
        _lib._lib = saved


# ------------------------------------------------------------------ fa2_bwd
DQ, DK, DV, DELTA, OO, DOUT = 6 << 20, 7 << 20, 8 << 20, 9 << 20, 10 << 20, 11 << 20


def bcall(q=Q, k=K, v=V, o=OO, lse=L, dout=DOUT, dq=DQ, dk=DK, dv=DV, delta=DELTA, **kw):
    a = dict(GOOD, **kw)
    return fa2.fa2_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, a["B"], a["H"], a["N"], a["d"],
                       a["scale"], a["causal"], 0)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta"])
def test_bwd_null_pointer(lib, which):
    assert bcall(**{which: 0}) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [0, 16, 63, 160, 256, 512])
def test_bwd_unsupported_head_dim(lib, d):
    assert bcall(d=d) == fa2.FA2_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=-1), dict(N=0), dict(N=(1 << 22) + 1),
                                dict(scale=math.inf), dict(scale=math.nan)])
def test_bwd_bad_sizes(lib, kw):
    assert bcall(**kw) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["q", "dout", "dq", "dv", "delta", "lse"])
def test_bwd_misaligned(lib, which):
    base = dict(q=Q, k=K, v=V, o=OO, lse=L, dout=DOUT, dq=DQ, dk=DK, dv=DV, delta=DELTA)
    assert bcall(**{which: base[which] + 4}) == fa2.FA2_ERR_MISALIGNED


@pytest.mark.parametrize("out,onto", [("dq", "q"), ("dk", "o"), ("dv", "dout"), ("delta", "lse"),
                                      ("dq", "dk"), ("delta", "dv"), ("dk", "k")])
def test_bwd_output_overlap_rejected(lib, out, onto):
    base = dict(q=Q, k=K, v=V, o=OO, lse=L, dout=DOUT, dq=DQ, dk=DK, dv=DV, delta=DELTA)
    assert bcall(**{out: base[onto] + 16}) == fa2.FA2_ERR_INVALID_ARG


def test_bwd_inputs_may_alias_each_other(lib):
    # q = k = v is a valid call; with a misaligned delta (checked after the
    # overlap rules are reachable only for valid pointers) it stops before HIP.
    assert bcall(k=Q, v=Q, delta=DELTA + 4) == fa2.FA2_ERR_MISALIGNED


# ------------------------------------------------------------------ fa1_fwd
WS = 12 << 20


def fcall(q=Q, k=K, v=V, o=O, lse=L, ws=WS, ws_bytes=None, **kw):
    a = dict(GOOD, **kw)
    if ws_bytes is None:
        ws_bytes = fa2.fa1_workspace_bytes(a["B"], a["H"], a["N"], a["d"])
    return fa2.fa1_fwd(q, k, v, o, lse, ws, ws_bytes, a["B"], a["H"], a["N"], a["d"], a["scale"],
                       a["causal"], 0)


def test_fa1_workspace_size():
    assert fa2.fa1_workspace_bytes(2, 3, 100, 64) == 2 * 3 * 100 * 66 * 4
    assert fa2.fa1_workspace_bytes(0, 3, 100, 64) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d=128), "FA2_ERR_UNSUPPORTED"), (dict(d=32), "FA2_ERR_UNSUPPORTED"),
    (dict(ws=0), "FA2_ERR_INVALID_ARG"), (dict(ws_bytes=100), "FA2_ERR_INVALID_ARG"),
    (dict(N=(1 << 21) + 64), "FA2_ERR_INVALID_ARG"), (dict(ws=WS + 4), "FA2_ERR_MISALIGNED"),
    (dict(ws=Q + 16), "FA2_ERR_INVALID_ARG"), (dict(ws=O + 16), "FA2_ERR_INVALID_ARG"),
    (dict(scale=math.nan), "FA2_ERR_INVALID_ARG")])
def test_fa1_rejects(lib, kw, status):
    assert fcall(**kw) == getattr(fa2, status)


# --------------------------------------------------- fa2_fwd_splitkv / merge
@pytest.mark.parametrize("B,H,Nq,Nk,d,req", [(1, 32, 1, 65536, 128, 0), (1, 1, 1, 100, 64, 3),
                                             (2, 3, 5, 1000, 64, 7), (1, 2, 3, 640, 32, 6),
                                             (4, 32, 1, 4096, 64, 0), (1, 1, 200, 64, 96, 0),
                                             (1, 1, 1, 1, 128, 0), (1, 4, 7, 5000, 128, 4096)])
def test_split_plan_has_no_empty_range(lib, B, H, Nq, Nk, d, req):
    n = fa2.fa2_splitkv_splits(B, H, Nq, Nk, d, req)
    tiles = -(-Nk // 64)
    assert 1 <= n <= tiles
    if req:
        assert n <= req
    tps = -(-tiles // n)
    assert (n - 1) * tps < tiles <= n * tps
    ws = fa2.fa2_splitkv_workspace_bytes(B, H, Nq, Nk, d, req)
    assert ws == (0 if n == 1 else n * B * H * Nq * (d + 1) * 4)


def test_split_plan_auto_fills_the_chip():
    # one query row per head, 32 heads, 64K keys: 8 ranges of 128 tiles, so
    # 256 workgroups (one per CU); 256 heads need no split
    assert fa2.fa2_splitkv_splits(1, 32, 1, 65536, 128, 0) == 8
    assert fa2.fa2_splitkv_splits(8, 32, 1, 8192, 128, 0) == 1
    assert fa2.fa2_splitkv_splits(1, 8, 1, 131072, 128, 0) == 32
    assert fa2.fa2_splitkv_splits(1, 32, 1, 65536, 128, 1) == 1
    assert fa2.fa2_splitkv_splits(1, 32, 1, 65536, 128, -1) == 0


def scall(q=Q, k=K, v=V, o=O, lse=L, ws=WS, ws_bytes=None, B=1, H=2, Nq=3, Nk=1000, d=64,
          scale=0.125, n_splits=4):
    if ws_bytes is None:
        ws_bytes = fa2.fa2_splitkv_workspace_bytes(B, H, Nq, Nk, d, n_splits)
    return fa2.fa2_fwd_splitkv(q, k, v, o, lse, ws, ws_bytes, B, H, Nq, Nk, d, scale, n_splits, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), "FA2_ERR_INVALID_ARG"), (dict(Nq=0), "FA2_ERR_INVALID_ARG"),
    (dict(Nk=0), "FA2_ERR_INVALID_ARG"), (dict(Nk=(1 << 22) + 1), "FA2_ERR_INVALID_ARG"),
    (dict(d=256), "FA2_ERR_UNSUPPORTED"), (dict(d=48), "FA2_ERR_UNSUPPORTED"),
    (dict(n_splits=-1), "FA2_ERR_INVALID_ARG"), (dict(n_splits=5000), "FA2_ERR_INVALID_ARG"),
    (dict(scale=math.inf), "FA2_ERR_INVALID_ARG"), (dict(ws=0), "FA2_ERR_INVALID_ARG"),
    (dict(ws_bytes=64), "FA2_ERR_INVALID_ARG"), (dict(ws=WS + 8), "FA2_ERR_MISALIGNED"),
    (dict(o=Q + 16), "FA2_ERR_INVALID_ARG"), (dict(ws=K + 16), "FA2_ERR_INVALID_ARG"),
    (dict(lse=O + 16), "FA2_ERR_INVALID_ARG")])
def test_splitkv_rejects(lib, kw, status):
    assert scall(**kw) == getattr(fa2, status)


def test_splitkv_single_range_needs_no_workspace(lib):
    # one range: ws may be NULL; a misaligned q proves the call got past the
    # workspace rules without reaching HIP
    assert fa2.fa2_splitkv_workspace_bytes(1, 2, 3, 1000, 64, 1) == 0
    assert scall(ws=0, ws_bytes=0, n_splits=1, q=Q + 2) == fa2.FA2_ERR_MISALIGNED


@pytest.mark.parametrize("kw,status", [
    (dict(op=0), "FA2_ERR_INVALID_ARG"), (dict(n=0), "FA2_ERR_INVALID_ARG"),
    (dict(rows=0), "FA2_ERR_INVALID_ARG"), (dict(d=256), "FA2_ERR_UNSUPPORTED"),
    (dict(o=Q + 8), "FA2_ERR_MISALIGNED"), (dict(o=Q + 16), "FA2_ERR_INVALID_ARG"),
    (dict(lse=K + 16), "FA2_ERR_INVALID_ARG"), (dict(lse=O + 16), "FA2_ERR_INVALID_ARG")])
def test_lse_merge_rejects(lib, kw, status):
    a = dict(op=Q, lp=K, o=O, lse=L, n=4, rows=100, d=64)
    a.update(kw)
    assert fa2.fa2_lse_merge(a["op"], a["lp"], a["o"], a["lse"], a["n"], a["rows"], a["d"], 0) == \
        getattr(fa2, status)


def test_fa1_workspace_size_rejects_huge_grids():
    assert fa2.fa1_workspace_bytes(1 << 16, 1 << 16, 1, 64) == 0


# --------------------------------------------------- fa2_fwd_splitkv_noalloc
def ncall(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Nq=3, Nk=1000, d=64, scale=0.125, n_splits=4):
    return fa2.fa2_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, n_splits, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), "FA2_ERR_INVALID_ARG"), (dict(lse=0), "FA2_ERR_INVALID_ARG"),
    (dict(Nq=0), "FA2_ERR_INVALID_ARG"), (dict(Nk=(1 << 22) + 1), "FA2_ERR_INVALID_ARG"),
    (dict(d=256), "FA2_ERR_UNSUPPORTED"), (dict(n_splits=-1), "FA2_ERR_INVALID_ARG"),
    (dict(n_splits=5000), "FA2_ERR_INVALID_ARG"), (dict(scale=math.nan), "FA2_ERR_INVALID_ARG"),
    (dict(k=K + 8), "FA2_ERR_MISALIGNED"), (dict(o=Q + 16), "FA2_ERR_INVALID_ARG"),
    (dict(lse=O + 16), "FA2_ERR_INVALID_ARG"), (dict(o=V), "FA2_ERR_INVALID_ARG")])
def test_noalloc_rejects(lib, kw, status):
    assert ncall(**kw) == getattr(fa2, status)


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    # 4096 ranges x 64 heads x 129 floats of partial results: 135 MB, more
    # than the fixed 8 MiB; the same call with a workspace is valid
    a = dict(B=1, H=64, Nq=1, Nk=4096 * 64, d=128, n_splits=4096)
    need = fa2.fa2_splitkv_workspace_bytes(a["B"], a["H"], a["Nq"], a["Nk"], a["d"], 4096)
    assert need == 4096 * 64 * 129 * 4 > fa2.FA2_NOALLOC_SCRATCH_BYTES
    far = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, lse=5 << 40)   # 4.3 GB K and V
    assert ncall(**far, **a) == fa2.FA2_ERR_SCRATCH_LIMIT
    assert "fixed buffer" in fa2.fa2_status_string(fa2.FA2_ERR_SCRATCH_LIMIT)
    # the argument checks come first
    assert ncall(**dict(far, o=(2 << 40) + 64), **a) == fa2.FA2_ERR_INVALID_ARG
    assert ncall(**far, **dict(a, d=48)) == fa2.FA2_ERR_UNSUPPORTED


def test_noalloc_scratch_covers_the_decode_workloads():
    # every decoding workload, with the library's split count, fits the
    # fixed scratch (so the no-allocation entry point serves them)
    from exact_attention_fwd_amd.workloads import WORKLOADS
    for w in WORKLOADS.values():
        if w.Nq:
            assert fa2.fa2_splitkv_workspace_bytes(w.B, w.H, w.nq, w.N, w.d, 0) <= \
                fa2.FA2_NOALLOC_SCRATCH_BYTES, w.name
