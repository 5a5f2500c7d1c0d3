"""fa2_fwd_splitkv_noalloc on the GPU, through the C ABI: the entry point
that allocates nothing (its partial results go to the library's fixed
scratch buffer) gives exactly what fa2_fwd_splitkv gives with a caller
workspace, on several calls in a row -- a large one, a smaller one, the
large one again -- so the shared buffer's leftover contents from one call
never reach the next; and it meets the forward's gates against the float64
oracle.  Collected last: it is the only test that touches the buffer.
"""
import numpy as np
import pytest

from exact_attention_fwd_amd.workloads import make_qkv, sample_rows
from oracle import attention_fp64
from parity import diff, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(B, H, Nq, Nk, d, seed):
    q = make_qkv(B, H, Nq, d, 1.0, seed)[0]
    _, k, v = make_qkv(B, H, Nk, d, 1.0, seed + 1)
    return q, k, v


# (B, H, Nq, Nk, d): 32 query rows per head against a 64K cache (8 key
# ranges, 4.2 MB of partial results), then a smaller ragged call (16 ranges,
# 100 KB), then the first again.
CALLS = [(1, 32, 32, 65536, 128), (2, 4, 3, 5000, 64), (1, 32, 32, 65536, 128)]


def test_noalloc_matches_the_workspace_entry_point_call_after_call():
    import exact_attention_fwd_amd as fa2

    dev = torch.device("cuda:0")
    for i, (B, H, Nq, Nk, d) in enumerate(CALLS):
        name = f"call {i}: [{B},{H},{Nq}|{Nk},{d}]"
        say(f"[noalloc] {name}")
        n_splits = fa2.fa2_splitkv_splits(B, H, Nq, Nk, d, 0)
        need = fa2.fa2_splitkv_workspace_bytes(B, H, Nq, Nk, d, 0)
        assert n_splits > 1 and 0 < need <= fa2.FA2_NOALLOC_SCRATCH_BYTES, name
        q, k, v = _inputs(B, H, Nq, Nk, d, seed=i % 2)
        tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        o_ws, l_ws = fa2.fwd_splitkv(tq, tk, tv, scale=d ** -0.5)
        # poisoned outputs: every element must be written
        o_na = torch.full_like(tq, float("nan"))
        l_na = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
        fa2.fwd_splitkv_noalloc(tq, tk, tv, o_na, l_na, scale=d ** -0.5)
        torch.cuda.synchronize(dev)
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), name
        assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32)), name
        # the forward's gates against the oracle (every row of the small
        # call, 64 seeded rows per head of the large one)
        o, l = o_na.cpu().numpy(), l_na.cpu().numpy()
        if Nq <= 8:
            o_ref, l_ref = attention_fp64(q, k, v, d ** -0.5)
            dd = diff(o, l, o_ref, l_ref)
        else:
            rows = np.stack([np.stack([sample_rows(Nq, b, h, 8) for h in range(H)])
                             for b in range(B)])
            o_ref, l_ref = attention_fp64(q, k, v, d ** -0.5, rows=rows)
            bi = np.arange(B)[:, None, None]
            hi = np.arange(H)[None, :, None]
            dd = diff(o[bi, hi, rows], l[bi, hi, rows], o_ref, l_ref)
        say(f"[noalloc] {name}: {n_splits} ranges, {need} B of scratch, bit-identical; {dd}")
        assert dd.ok(), f"{name}: {dd}"


def test_noalloc_on_the_null_stream_and_a_side_stream():
    """The buffer address is per device, whatever stream the call uses."""
    import exact_attention_fwd_amd as fa2

    dev = torch.device("cuda:0")
    B, H, Nq, Nk, d = 1, 8, 1, 20000, 128
    q, k, v = _inputs(B, H, Nq, Nk, d, seed=5)
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o_ws, l_ws = fa2.fwd_splitkv(tq, tk, tv)
    torch.cuda.synchronize(dev)
    side = torch.cuda.Stream(dev)
    for stream in (0, side.cuda_stream):
        o = torch.empty_like(tq)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
        torch.cuda.synchronize(dev)
        fa2.fwd_splitkv_noalloc(tq, tk, tv, o, lse, stream=stream)
        torch.cuda.synchronize(dev)
        assert torch.equal(o.view(torch.int16), o_ws.view(torch.int16)), stream
        assert torch.equal(lse.view(torch.int32), l_ws.view(torch.int32)), stream
