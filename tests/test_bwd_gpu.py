"""GPU parity of the backward pass: fa2_bwd's dQ, dK, dV and delta against the
float64 gradient oracle, on the same seeded inputs, through the C ABI.

The GPU forward supplies O and LSE (as a caller would); the oracle works
from Q, K, V and dO alone, so the gates cover the forward's rounding too.
Gates (tests/parity.py): per tensor, the error in units of its worst-case
rounding bound u (|G| + E + 2^-14) is at most 2 everywhere, and its rms at
most the rms of the statistical bound (u / sqrt 3) S (E and S from the
oracle's error-scale functions).  Run on the oracle's own O and LSE (rounded
to fp16 and fp32, as the forward hands them over), delta must also meet its
definition dO . O for that O within the fp32 bound.  Cases: odd N at every supported head dim, causal
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
from oracle import attention_fp64
from oracle.attention_bwd import attention_bwd_error_scale, attention_bwd_error_std
from parity import delta_contract, grad_diff, run_gpu_bwd, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BWD_HEAD_DIMS = [32, 64, 96, 128]


def _do(shape, seed):
    """Upstream gradient: i.i.d. N(0, 1) in fp16, its own seed."""
    return make_qkv(*shape, 1.0, seed=seed + 7919)[0]


def check_bwd(name, q, k, v, do, scale, causal, given_o=False):
    """The GPU backward against the oracle.  given_o: run it on the oracle's
    O and LSE (rounded as the forward stores them) instead of the GPU
    forward's, and check delta against its definition for that O."""
    o16 = lse32 = None
    if given_o:
        o_ref, l_ref = attention_fp64(q, k, v, scale, causal=causal)
        o16, lse32 = o_ref.astype(np.float16), l_ref.astype(np.float32)
    got = run_gpu_bwd(q, k, v, do, scale, causal, o=o16, lse=lse32)
    ref = attention_bwd_fp64(q, k, v, do, scale, causal=causal)
    esc = attention_bwd_error_scale(q, k, v, do, scale, causal=causal)
    sd = attention_bwd_error_std(q, k, v, do, scale, causal=causal)
    msgs, ok = [], True
    for label, g, r, e, sg in zip(("dq", "dk", "dv", "delta"), got, ref, esc, sd):
        assert np.all(np.isfinite(g.astype(np.float32))), f"{name}: {label} not finite"
        dd = grad_diff(g, r, e, sg)
        msgs.append(f"{label} {dd}")
        ok &= dd.ok()
    if given_o:
        dc = delta_contract(got[3], do, o16)
        msgs.append(f"delta vs dO.O {dc:.3f}")
        ok &= dc <= 1.0
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
    sd = attention_bwd_error_std(q, k, v, do, d ** -0.5, causal=True)
    for g, r, e, sg in zip((dq, dk, dv, delta), ref, esc, sd):
        assert grad_diff(g.cpu().numpy(), r, e, sg).ok()


@pytest.mark.parametrize("d", BWD_HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [17, 129, 300])
def test_on_the_oracles_o_and_lse(n, d, causal):
    """The backward's own arithmetic: O and LSE from the oracle, so the only
    roundings are the backward's; delta checked against dO . O for that O."""
    q, k, v = make_qkv(1, 2, n, d, 1.0, seed=n + 1)
    check_bwd(f"given O: N={n} d={d} causal={causal}", q, k, v, _do(q.shape, n + 1), d ** -0.5,
              causal, given_o=True)


@pytest.mark.parametrize("causal", [False, True])
def test_on_the_oracles_o_full_size(causal):
    shape = (2, 16, 2048, 64)
    q, k, v = make_qkv(*shape, 1.0, seed=0)
    check_bwd(f"given O: {list(shape)} causal={causal}", q, k, v, _do(shape, 0), 0.125, causal,
              given_o=True)


def test_head_dim_256_is_rejected():
    import exact_attention_fwd_amd as fa2
    q = torch.zeros((1, 1, 64, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.bwd(q, q, q, q.clone(), torch.zeros((1, 1, 64), device="cuda"), q.clone())
    assert e.value.status == fa2.FA2_ERR_UNSUPPORTED
