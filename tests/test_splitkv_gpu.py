"""GPU parity of the split key/value forward (fa2_fwd_splitkv) and of the
merge (fa2_lse_merge) against the float64 oracle, through the C ABI.

fa2_fwd_splitkv computes the same function as the forward (non-causal),
for Nq queries over Nk keys, so it is held to the forward's gates
(tests/parity.py) against ``attention_fp64`` with Nq != Nk.  Cases: one
query (decoding) to a few hundred, key counts with tails inside a 64-key
tile and inside a range, every supported head dim, one range / several /
the library's choice / more ranges than tiles, a long cache
[1,32,1,65536,128], scale 0 and negative, and results that do not depend
on the split beyond the tolerance.  fa2_lse_merge is checked against
``merge_lse_fp64`` on random parts, with empty parts (LSE = -inf holding
garbage) and LSE values far beyond exp's range.
"""
import numpy as np
import pytest

from exact_attention_fwd_amd.workloads import make_qkv
from oracle import attention_fp64, merge_lse_fp64
from parity import diff, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(B, H, Nq, Nk, d, seed, sigma=1.0):
    q = make_qkv(B, H, Nq, d, sigma, seed)[0]
    _, k, v = make_qkv(B, H, Nk, d, sigma, seed + 1)
    return q, k, v


def run_splitkv(q, k, v, scale, n_splits):
    import exact_attention_fwd_amd as fa2
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v))
    o, l = fa2.fwd_splitkv(tq, tk, tv, scale=scale, n_splits=n_splits)
    torch.cuda.synchronize()
    return o.cpu().numpy(), l.cpu().numpy()


def check(name, q, k, v, scale, n_splits):
    o, l = run_splitkv(q, k, v, scale, n_splits)
    assert np.all(np.isfinite(o.astype(np.float32))) and np.all(np.isfinite(l)), name
    o_ref, l_ref = attention_fp64(q, k, v, scale)
    dd = diff(o, l, o_ref, l_ref)
    say(f"[splitkv parity] {name}: {dd}")
    assert dd.ok(), f"{name}: {dd}"
    return o, l


@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 63), (1, 65), (5, 1000), (32, 4096), (33, 700),
                                   (100, 2000)])
@pytest.mark.parametrize("n_splits", [1, 0, 3])
def test_shapes_and_splits(d, nq, nk, n_splits):
    q, k, v = _inputs(1, 2, nq, nk, d, seed=nq * 7 + nk)
    check(f"Nq={nq} Nk={nk} d={d} splits={n_splits}", q, k, v, d ** -0.5, n_splits)


def test_more_ranges_than_tiles_and_batches():
    q, k, v = _inputs(3, 4, 2, 300, 64, seed=5)
    for n in (1, 2, 5, 64):
        check(f"[3,4,2|300,64] splits={n}", q, k, v, 0.125, n)


def test_long_cache_decode():
    q, k, v = _inputs(1, 32, 1, 65536, 128, seed=9, sigma=0.5)
    o0, l0 = check("[1,32,1|65536,128] auto", q, k, v, 128 ** -0.5, 0)
    o1, l1 = check("[1,32,1|65536,128] one range", q, k, v, 128 ** -0.5, 1)
    assert np.abs(o0.astype(np.float32) - o1.astype(np.float32)).max() <= 4e-3


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3])
def test_scale_values(scale):
    q, k, v = _inputs(1, 2, 3, 777, 64, seed=11)
    check(f"scale={scale}", q, k, v, scale, 0)


def test_merge_against_the_oracle():
    import exact_attention_fwd_amd as fa2
    rng = np.random.default_rng(3)
    S, rows, d = 6, 300, 128
    o_parts = rng.standard_normal((S, rows, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((S, rows)) * 5).astype(np.float32)
    lse_parts[2, :50] = -np.inf               # empty parts holding garbage
    o_parts[2, :50] = 1e30
    lse_parts[:, 50:60] = -np.inf             # rows with no keys at all
    lse_parts[:, 60:70] += 900.0              # far beyond exp's range
    o, l = fa2.lse_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda())
    torch.cuda.synchronize()
    o, l = o.cpu().numpy(), l.cpu().numpy()
    o_ref, l_ref = merge_lse_fp64(o_parts, lse_parts)
    keep = np.isfinite(l_ref)
    assert np.all(o[~keep] == 0) and np.all(l[~keep] == -np.inf)
    dd = diff(o[keep], l[keep], o_ref[keep], l_ref[keep])
    say(f"[merge parity] {dd}")
    assert dd.ok(), str(dd)


def test_merge_of_gpu_parts_equals_full_attention():
    """Attend to two key halves with one range each, merge on the GPU, and
    compare with the oracle over all keys: the merge as a building block of
    key-sharded attention."""
    import exact_attention_fwd_amd as fa2
    q, k, v = _inputs(2, 4, 16, 1500, 64, seed=13)
    parts = []
    for a, b in ((0, 700), (700, 1500)):
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).cuda()
                      for x in (q, k[:, :, a:b], v[:, :, a:b]))
        o, l = fa2.fwd_splitkv(tq, tk, tv, scale=0.125, n_splits=1)
        parts.append((o.float(), l))
    o_p = torch.stack([p[0] for p in parts]).contiguous()
    l_p = torch.stack([p[1] for p in parts]).contiguous()
    o, l = fa2.lse_merge(o_p, l_p)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_fp64(q, k, v, 0.125)
    dd = diff(o.cpu().numpy(), l.cpu().numpy(), o_ref, l_ref)
    say(f"[merge of gpu parts] {dd}")
    assert dd.ok(), str(dd)
