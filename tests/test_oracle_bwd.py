"""Pins of the float64 gradient oracle (``oracle.attention_bwd``), CPU only.

The gradient formulas are pinned to things other than themselves:
  * central finite differences of the forward oracle (already pinned to the
    pages' worked examples) along random directions;
  * torch autograd, in float64 on the CPU, of an independently written
    forward;
  * exact identities of the function: shifting every key by one vector
    leaves each row's softmax unchanged (sum_j dK_j = 0); every row of P
    sums to one (sum_j dV_j = sum_i dO_i); scaling Q or K by t is the same
    map, so <dQ, Q> = <dK, K>; delta_i = dO_i . O_i;
  * special cases: N = 1, the causal first row, Q = 0 (uniform weights),
    a constant V.
A last test plants mistakes in the oracle (a dropped term, a wrong sign, a
missing scale, a transposed operand) and shows each one fails a pin.
"""
import numpy as np
import pytest

import oracle.attention_bwd as ob
from oracle import attention_bwd_fp64, attention_fp64

SCALE = 0.375   # exactly representable in fp32


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _case(N=9, d=6, B=1, H=2, seed=0):
    q = _rand((B, H, N, d), seed)
    k = _rand((B, H, N, d), seed + 1)
    v = _rand((B, H, N, d), seed + 2)
    do = _rand((B, H, N, d), seed + 3)
    return q, k, v, do


def _loss(q, k, v, do, causal):
    o, _ = attention_fp64(q, k, v, SCALE, causal=causal, threads=1)
    return float((o * do).sum())


def _fd_errors(q, k, v, do, causal, grads, n_dirs=3, h=1e-6):
    """Relative error of <G, E> against the central difference along E."""
    errs = []
    rng = np.random.default_rng(123)
    for which in range(3):
        for _ in range(n_dirs):
            e = rng.standard_normal(q.shape)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = args_p[which] + h * e
            args_m[which] = args_m[which] - h * e
            fd = (_loss(*args_p, do, causal) - _loss(*args_m, do, causal)) / (2 * h)
            an = float((grads[which] * e).sum())
            errs.append(abs(fd - an) / max(1.0, abs(fd)))
    return max(errs)


def _identity_errors(q, k, v, do, causal, dq, dk, dv, delta):
    o, _ = attention_fp64(q, k, v, SCALE, causal=causal, threads=1)
    e1 = np.abs(dk.sum(axis=2)).max()                                  # sum_j dK_j = 0
    e2 = np.abs(dv.sum(axis=2) - do.sum(axis=2)).max()                 # sum_j dV_j = sum_i dO_i
    e3 = abs((dq * q).sum() - (dk * k).sum())                          # <dQ,Q> = <dK,K>
    e4 = np.abs(delta - (do * o).sum(axis=-1)).max()                   # delta = dO . O
    return max(e1, e2, e3, e4)


def _torch_grads(q, k, v, do, causal):
    torch = pytest.importorskip("torch")
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = SCALE * torch.matmul(qt, kt.transpose(-1, -2).contiguous())
    if causal:
        n = q.shape[2]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vt)
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_finite_differences(causal):
    q, k, v, do = _case()
    dq, dk, dv, _ = attention_bwd_fp64(q, k, v, do, SCALE, causal=causal, threads=1)
    assert _fd_errors(q, k, v, do, causal, (dq, dk, dv)) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 4), (7, 3), (33, 16)])
def test_gradients_match_torch_autograd(causal, N, d):
    q, k, v, do = _case(N=N, d=d, seed=N)
    dq, dk, dv, _ = attention_bwd_fp64(q, k, v, do, SCALE, causal=causal, threads=1)
    tq, tk, tv = _torch_grads(q, k, v, do, causal)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    q, k, v, do = _case(N=40, d=8, seed=5)
    dq, dk, dv, delta = attention_bwd_fp64(q, k, v, do, SCALE, causal=causal, threads=1)
    assert _identity_errors(q, k, v, do, causal, dq, dk, dv, delta) < 1e-10


def test_single_key_passes_do_to_dv_and_nothing_to_q_k():
    q, k, v, do = _case(N=1, d=5)
    for causal in (False, True):
        dq, dk, dv, _ = attention_bwd_fp64(q, k, v, do, SCALE, causal=causal, threads=1)
        assert np.all(dq == 0) and np.all(dk == 0)
        np.testing.assert_array_equal(dv, do)


def test_causal_first_row_has_no_query_gradient():
    q, k, v, do = _case(N=12, d=4, seed=9)
    dq, _, _, _ = attention_bwd_fp64(q, k, v, do, SCALE, causal=True, threads=1)
    assert np.all(dq[:, :, 0] == 0)
    assert np.abs(dq[:, :, 1:]).max() > 1e-3


def test_zero_queries_uniform_weights_closed_form():
    """Q = 0: P = 1/N, so dV_j = mean_i dO_i for every j, dK = 0 (dK is a sum
    of dS times Q), and dQ_i = (sigma/N) sum_j (dO_i . (V_j - mean V)) K_j."""
    q, k, v, do = _case(N=10, d=6, seed=3)
    q[:] = 0
    dq, dk, dv, _ = attention_bwd_fp64(q, k, v, do, SCALE, causal=False, threads=1)
    N = q.shape[2]
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape),
                               rtol=1e-12, atol=1e-14)
    assert np.abs(dk).max() == 0
    vc = v - v.mean(axis=2, keepdims=True)
    want = SCALE / N * np.einsum("bhic,bhjc,bhjd->bhid", do, vc, k)
    np.testing.assert_allclose(dq, want, rtol=1e-10, atol=1e-13)


def test_constant_values_give_no_query_or_key_gradient():
    """V_j = w for all j: O_i = w whatever P is, so dQ = dK = 0 and
    dV_j = sum_i P_ij dO_i."""
    q, k, v, do = _case(N=16, d=5, seed=4)
    v[:] = v[:, :, :1]
    for causal in (False, True):
        dq, dk, dv, _ = attention_bwd_fp64(q, k, v, do, SCALE, causal=causal, threads=1)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12)


def test_row_blocks_and_threads_do_not_change_results():
    q, k, v, do = _case(N=50, d=8, B=2, H=3, seed=8)
    ref = attention_bwd_fp64(q, k, v, do, SCALE, causal=True, threads=1, row_block=50)
    for rb, th in ((1, 1), (7, 4), (16, 8)):
        got = attention_bwd_fp64(q, k, v, do, SCALE, causal=True, threads=th, row_block=rb)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_planted_mistakes_fail_a_pin(monkeypatch):
    """Each plausible slip in the chain rule is caught by finite differences
    or by an identity."""
    q, k, v, do = _case(N=9, d=6, seed=11)
    good = ob._bwd_rows

    def drop_delta(q_rows, row_ids, k, v, do_rows, sigma, causal):
        s = ob._masked_scores(q_rows, row_ids, k, sigma, causal)
        _, e, l = ob._stable_softmax_parts(s)
        p = e / l[:, None]
        dp = do_rows @ v.T
        ds = p * dp
        return sigma * (ds @ k), sigma * (ds.T @ q_rows), p.T @ do_rows, (p * dp).sum(1)

    def flip_dq(*a):
        dq, dk, dv, dl = good(*a)
        return -dq, dk, dv, dl

    def no_scale_dk(q_rows, row_ids, k, v, do_rows, sigma, causal):
        dq, dk, dv, dl = good(q_rows, row_ids, k, v, do_rows, sigma, causal)
        return dq, dk / sigma, dv, dl

    def transposed_dv(q_rows, row_ids, k, v, do_rows, sigma, causal):
        s = ob._masked_scores(q_rows, row_ids, k, sigma, causal)
        _, e, l = ob._stable_softmax_parts(s)
        p = e / l[:, None]
        dq, dk, _, dl = good(q_rows, row_ids, k, v, do_rows, sigma, causal)
        return dq, dk, p @ do_rows, dl

    for causal in (False, True):
        for bad in (drop_delta, flip_dq, no_scale_dk, transposed_dv):
            monkeypatch.setattr(ob, "_bwd_rows", bad)
            dq, dk, dv, delta = ob.attention_bwd_fp64(q, k, v, do, SCALE, causal=causal, threads=1)
            monkeypatch.setattr(ob, "_bwd_rows", good)
            fd = _fd_errors(q, k, v, do, causal, (dq, dk, dv), n_dirs=1)
            ident = _identity_errors(q, k, v, do, causal, dq, dk, dv, delta)
            assert fd > 1e-3 or ident > 1e-3, (bad.__name__, causal, fd, ident)
