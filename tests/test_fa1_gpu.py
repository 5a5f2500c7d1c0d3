"""GPU parity of the FlashAttention-1-order comparator (fa1_fwd) against the
float64 oracle, at the forward's gates (tests/parity.py), through the C ABI.

The comparator computes the same function as fa2_fwd in another loop order
(one workgroup per head, key/value blocks outside, the normalised fp32
output and (m, l) written back after every block), so it is held to the
same tolerance.  Cases: the reference shape [4,32,2048,64] non-causal and
causal, odd N (tails inside the 128-key blocks and the 128-query steps),
batch x heads, stress inputs that move the row max between blocks, scale
values, and agreement with fa2_fwd on the reference shape.
"""
import numpy as np
import pytest

from exact_attention_fwd_amd.workloads import WORKLOADS, make_qkv, stress_inputs
from oracle import attention_fp64
from parity import diff, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run_fa1(q, k, v, scale, causal):
    import exact_attention_fwd_amd as fa2
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v))
    o, l = fa2.fwd_fa1(tq, tk, tv, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu().numpy(), l.cpu().numpy()


def check(name, q, k, v, scale, causal):
    o, l = run_fa1(q, k, v, scale, causal)
    assert np.all(np.isfinite(o.astype(np.float32))) and np.all(np.isfinite(l)), name
    o_ref, l_ref = attention_fp64(q, k, v, scale, causal=causal)
    dd = diff(o, l, o_ref, l_ref)
    say(f"[fa1 parity] {name}: {dd}")
    assert dd.ok(), f"{name}: {dd}"
    return o, l


@pytest.mark.parametrize("causal", [False, True])
def test_reference_shape(causal):
    w = WORKLOADS["ref"]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    check(f"ref causal={causal}", q, k, v, w.scale, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 5, 64, 127, 128, 129, 255, 300, 1000])
def test_odd_lengths(n, causal):
    q, k, v = make_qkv(1, 2, n, 64, 1.0, seed=n)
    check(f"N={n} causal={causal}", q, k, v, 0.125, causal)


def test_batch_heads():
    q, k, v = make_qkv(3, 5, 300, 64, 1.0, seed=7)
    for causal in (False, True):
        check(f"[3,5,300,64] causal={causal}", q, k, v, 0.125, causal)


@pytest.mark.parametrize("kind", ["rising", "falling", "large", "const_v", "zero_q"])
@pytest.mark.parametrize("causal", [False, True])
def test_stress(kind, causal):
    q, k, v = stress_inputs(kind, 1, 2, 333, 64, seed=3)
    check(f"stress {kind} causal={causal}", q, k, v, 1.0 if kind in ("rising", "falling") else 0.125,
          causal)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3])
def test_scale_values(scale):
    q, k, v = make_qkv(1, 2, 200, 64, 1.0, seed=11)
    for causal in (False, True):
        check(f"scale={scale} causal={causal}", q, k, v, scale, causal)


def test_agrees_with_fa2_within_the_tolerance():
    import exact_attention_fwd_amd as fa2
    w = WORKLOADS["ref"]
    q, k, v = (torch.from_numpy(x).cuda() for x in make_qkv(w.B, w.H, w.N, w.d, w.sigma, w.seed))
    for causal in (False, True):
        o1, l1 = fa2.fwd_fa1(q, k, v, causal=causal)
        o2, l2 = fa2.fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert (o1.float() - o2.float()).abs().max().item() <= 4e-3
        assert ((l1 - l2).abs() / l2.abs().clamp(min=1)).max().item() <= 1e-4
