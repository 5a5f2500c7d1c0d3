"""GPU parity of the backward pass: fa2_bwd's dQ, dK, dV and delta against the
float64 gradient oracle, on the same seeded inputs, through the C ABI.

The GPU forward supplies O and LSE (as a caller would); the oracle works
from Q, K, V and dO alone, so the gates cover the forward's rounding too.
Gates (tests/parity.py): per tensor, the error in units of its rounding
bound u (|G| + E + 2^-14) -- E the oracle's per-element error scale -- is at
most 2 everywhere and 0.5 in rms.  Cases: odd N at every supported head dim, causal
and not; batch x heads with a ragged tail; the reference shape
[4,32,2048,64] and [4,16,2048,128] (every element); long sequences, N = 8192
(every element of two heads); stress inputs that move
the row max or concentrate the weights; scale 0 / negative / small; closed
forms (Q = 0: dK = 0 exactly; N = 1: dV = dO exactly, dQ and dK ~ 0);
determinism and guard bands; d = 256 rejected.
"""
import numpy as np
import pytest

from exact_attention_fwd_amd.workloads import make_qkv, stress_inputs
from oracle import attention_bwd_fp64
from oracle.attention_bwd import attention_bwd_error_scale
from parity import grad_diff, run_gpu_bwd, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BWD_HEAD_DIMS = [32, 64, 96, 128]


def _do(shape, seed):
    """Upstream gradient: i.i.d. N(0, 1) in fp16, its own seed."""
    return make_qkv(*shape, 1.0, seed=seed + 7919)[0]


def check_bwd(name, q, k, v, do, scale, causal):
    got = run_gpu_bwd(q, k, v, do, scale, causal)
    ref = attention_bwd_fp64(q, k, v, do, scale, causal=causal)
    esc = attention_bwd_error_scale(q, k, v, do, scale, causal=causal)
    msgs, ok = [], True
    for label, g, r, e in zip(("dq", "dk", "dv", "delta"), got, ref, esc):
        assert np.all(np.isfinite(g.astype(np.float32))), f"{name}: {label} not finite"
        dd = grad_diff(g, r, e)
        msgs.append(f"{label} {dd}")
        ok &= dd.ok()
    say(f"[bwd parity] {name}: " + "; ".join(msgs))
    assert ok, f"{name}: " + "; ".join(msgs)
    return got


@pytest.mark.parametrize("d", BWD_HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 17, 64, 65, 129, 300, 1000])
def test_odd_lengths(n, d, causal):
    q, k, v = make_qkv(1, 2, n, d, 1.0, seed=n)
    check_bwd(f"N={n} d={d} causal={causal}", q, k, v, _do(q.shape, n), d ** -0.5, causal)


@pytest.mark.parametrize("d", BWD_HEAD_DIMS)
def test_batch_heads_and_ragged_tail_together(d):
    q, k, v = make_qkv(3, 5, 300, d, 1.0, seed=7)
    do = _do(q.shape, 7)
    for causal in (False, True):
        check_bwd(f"[3,5,300,{d}] causal={causal}", q, k, v, do, d ** -0.5, causal)


@pytest.mark.parametrize("shape,causal", [((4, 32, 2048, 64), False), ((4, 32, 2048, 64), True),
                                          ((4, 16, 2048, 128), False), ((4, 16, 2048, 128), True)])
def test_full_size(shape, causal):
    q, k, v = make_qkv(*shape, 1.0, seed=0)
    check_bwd(f"{list(shape)} causal={causal}", q, k, v, _do(shape, 0), shape[3] ** -0.5, causal)


@pytest.mark.parametrize("d,causal", [(64, False), (128, False), (128, True)])
def test_long_sequence(d, causal):
    """N = 8192: 128 tiles of 64 rows per head, so each kernel's loop runs 128
    (causal: up to 128) tiles and the causal grid deals one head at a time."""
    shape = (1, 2, 8192, d)
    q, k, v = make_qkv(*shape, 1.0, seed=5)
    check_bwd(f"{list(shape)} causal={causal}", q, k, v, _do(shape, 5), d ** -0.5, causal)


@pytest.mark.parametrize("kind", ["rising", "falling", "large", "const_v", "zero_q"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_stress(kind, d, causal):
    q, k, v = stress_inputs(kind, 1, 2, 333, d, seed=3)
    scale = 1.0 if kind in ("rising", "falling") else d ** -0.5
    check_bwd(f"stress {kind} d={d} causal={causal}", q, k, v, _do(q.shape, 3), scale, causal)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3, 1e-3])
def test_scale_values(scale):
    q, k, v = make_qkv(1, 2, 200, 64, 1.0, seed=11)
    for causal in (False, True):
        check_bwd(f"scale={scale} causal={causal}", q, k, v, _do(q.shape, 11), scale, causal)


def test_closed_forms():
    """Q = 0 gives dK = 0 exactly (every dS row multiplies a zero query).
    N = 1 gives P = 1, so dV = dO exactly (P rounds to 1.0 in fp16) and
    dQ = dK = sigma * (dP - delta) * (K or Q), where dP and delta are the same
    dot product dO . v summed in two orders: within a few fp32 ulps of 0."""
    q, k, v = make_qkv(1, 2, 256, 64, 1.0, seed=21)
    do = _do(q.shape, 21)
    _, dk, _, _ = run_gpu_bwd(np.zeros_like(q), k, v, do, 0.125, False)
    assert np.all(dk == 0)
    q1, k1, v1 = make_qkv(2, 3, 1, 128, 1.0, seed=22)
    do1 = _do(q1.shape, 22)
    for causal in (False, True):
        dq, dk, dv, _ = run_gpu_bwd(q1, k1, v1, do1, 128 ** -0.5, causal)
        assert np.array_equal(dv, do1)
        assert np.abs(dq.astype(np.float32)).max() < 1e-4 and np.abs(dk.astype(np.float32)).max() < 1e-4


def test_deterministic():
    q, k, v = make_qkv(2, 4, 777, 128, 1.0, seed=5)
    do = _do(q.shape, 5)
    for causal in (False, True):
        a = run_gpu_bwd(q, k, v, do, 128 ** -0.5, causal)
        b = run_gpu_bwd(q, k, v, do, 128 ** -0.5, causal)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_guard_bands_untouched():
    import exact_attention_fwd_amd as fa2
    B, H, N, d, guard = 1, 3, 257, 64, 512
    q, k, v = make_qkv(B, H, N, d, 1.0, seed=9)
    do = _do(q.shape, 9)
    tq, tk, tv, tdo = (torch.from_numpy(x).cuda() for x in (q, k, v, do))
    o, lse = fa2.fwd(tq, tk, tv, causal=True)
    n_t, n_l = B * H * N * d, B * H * N
    bufs = [torch.full((n_t + 2 * guard,), 7.0, dtype=torch.float16, device="cuda") for _ in range(3)]
    lbuf = torch.full((n_l + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    dq, dk, dv = (b[guard:guard + n_t].view(B, H, N, d) for b in bufs)
    delta = lbuf[guard:guard + n_l].view(B, H, N)
    fa2.bwd(tq, tk, tv, o, lse, tdo, causal=True, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for b, n in [(x, n_t) for x in bufs] + [(lbuf, n_l)]:
        assert torch.all(b[:guard] == 7) and torch.all(b[guard + n:] == 7)
    ref = attention_bwd_fp64(q, k, v, do, d ** -0.5, causal=True)
    esc = attention_bwd_error_scale(q, k, v, do, d ** -0.5, causal=True)
    for g, r, e in zip((dq, dk, dv, delta), ref, esc):
        assert grad_diff(g.cpu().numpy(), r, e).ok()


def test_head_dim_256_is_rejected():
    import exact_attention_fwd_amd as fa2
    q = torch.zeros((1, 1, 64, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.bwd(q, q, q, q.clone(), torch.zeros((1, 1, 64), device="cuda"), q.clone())
    assert e.value.status == fa2.FA2_ERR_UNSUPPORTED
