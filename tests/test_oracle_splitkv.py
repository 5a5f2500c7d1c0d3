"""Pins of the oracle pieces the split-key-value path is checked against
(CPU only): attention of a short query block over a longer key/value set,
and the merge of partial results over disjoint key parts.

* Nq != Nk (no mask) against the pure-Python brute force, and against the
  rows of the square computation (every row is independent of the others);
* the merge against the forward oracle itself: split the keys into parts
  in many ways (uneven, single keys, one part), attend to each part, merge,
  and get the attention over all keys back to 1e-12 -- the recurrence's
  independence of grouping and order ([Attn-I] 3.6.4);
* merge invariants: one part is the identity, the parts' order does not
  matter, a part with LSE = -inf is ignored, LSE values far beyond exp's
  range merge to the closed form (max shift).
"""
import numpy as np
import pytest

from oracle import attention_fp64, brute_force_attention, merge_lse_fp64


def _qkv(B, H, Nq, Nk, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, Nq, d)), rng.standard_normal((B, H, Nk, d)),
            rng.standard_normal((B, H, Nk, d)))


@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 7), (3, 5), (2, 9), (5, 2)])
def test_short_queries_against_brute_force(nq, nk):
    q, k, v = _qkv(1, 2, nq, nk, 4, seed=nq * 10 + nk)
    o, l = attention_fp64(q, k, v, 0.5)
    ob, lb = brute_force_attention(q, k, v, 0.5)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l, np.array(lb), rtol=1e-13, atol=1e-13)


def test_short_queries_are_rows_of_the_square_problem():
    q, k, v = _qkv(2, 3, 40, 40, 8, seed=1)
    o_full, l_full = attention_fp64(q, k, v, 0.35)
    rows = [0, 7, 39]
    o, l = attention_fp64(q[:, :, rows], k, v, 0.35)
    np.testing.assert_allclose(o, o_full[:, :, rows], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l, l_full[:, :, rows], rtol=1e-14, atol=1e-14)


def test_causal_needs_square_shapes():
    q, k, v = _qkv(1, 1, 3, 5, 4, seed=2)
    with pytest.raises(ValueError):
        attention_fp64(q, k, v, 0.5, causal=True)


def _parts(q, k, v, cuts, scale):
    o_p, l_p = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = attention_fp64(q, k[:, :, a:b], v[:, :, a:b], scale)
        o_p.append(o)
        l_p.append(l)
    return np.stack(o_p), np.stack(l_p)


@pytest.mark.parametrize("cuts", [[0, 50], [0, 25, 50], [0, 1, 2, 50], [0, 17, 18, 33, 49, 50],
                                  list(range(51))])
def test_merge_of_key_parts_is_the_full_attention(cuts):
    q, k, v = _qkv(2, 2, 3, 50, 16, seed=4)
    o_ref, l_ref = attention_fp64(q, k, v, 0.6)
    o_p, l_p = _parts(q, k, v, cuts, 0.6)
    o, l = merge_lse_fp64(o_p, l_p)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, rtol=1e-12, atol=1e-12)


def test_merge_invariants():
    q, k, v = _qkv(1, 2, 4, 30, 8, seed=5)
    o_p, l_p = _parts(q, k, v, [0, 4, 19, 30], 0.4)
    o, l = merge_lse_fp64(o_p, l_p)
    perm = [2, 0, 1]
    o2, l2 = merge_lse_fp64(o_p[perm], l_p[perm])
    np.testing.assert_allclose(o2, o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=1e-14, atol=1e-14)
    o1, l1 = merge_lse_fp64(o_p[:1], l_p[:1])
    np.testing.assert_allclose(o1, o_p[0], rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(l1, l_p[0])
    # an empty part (LSE = -inf) with garbage output changes nothing
    o3, l3 = merge_lse_fp64(np.concatenate([o_p, np.full_like(o_p[:1], 1e30)]),
                            np.concatenate([l_p, np.full_like(l_p[:1], -np.inf)]))
    np.testing.assert_allclose(o3, o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l3, l, rtol=1e-14, atol=1e-14)


def test_merge_far_beyond_exp_range():
    o_p = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    l_p = np.array([[800.0], [801.0]])
    o, l = merge_lse_fp64(o_p, l_p)
    w1 = 1.0 / (1.0 + np.e)
    np.testing.assert_allclose(o[0], [w1, 1 - w1], rtol=1e-14)
    np.testing.assert_allclose(l[0], 801.0 + np.log1p(np.exp(-1.0)), rtol=1e-15)
    o_e, l_e = merge_lse_fp64(np.zeros((2, 1, 3)), np.full((2, 1), -np.inf))
    assert np.all(o_e == 0) and np.all(l_e == -np.inf)


# ------------------------------------------------ planted mistakes fail a pin
def _merge_mutants():
    good = merge_lse_fp64   # bound now: the pins see the mutant under this name

    def no_max_shift(o_parts, lse_parts):
        o, lse = np.asarray(o_parts, float), np.asarray(lse_parts, float)
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            w = np.exp(lse)
            total = w.sum(axis=0)
            return (w[..., None] * o).sum(axis=0) / total[..., None], np.log(total)

    def lse_without_shift(o_parts, lse_parts):
        o, l = good(o_parts, lse_parts)
        m = np.asarray(lse_parts, float).max(axis=0)
        return o, l - np.where(np.isfinite(m), m, 0.0)

    def unnormalised_output(o_parts, lse_parts):
        lse = np.asarray(lse_parts, float)
        m = lse.max(axis=0)
        shift = np.where(np.isfinite(m), m, 0.0)
        w = np.exp(lse - shift)
        o, l = good(o_parts, lse_parts)
        return (w[..., None] * np.asarray(o_parts, float)).sum(axis=0), l

    def max_instead_of_logsumexp(o_parts, lse_parts):
        o, _ = good(o_parts, lse_parts)
        return o, np.asarray(lse_parts, float).max(axis=0)

    def reversed_weights(o_parts, lse_parts):
        lse = np.asarray(lse_parts, float)
        neg = good(o_parts, -lse)
        return neg[0], good(o_parts, lse_parts)[1]

    def plain_average(o_parts, lse_parts):
        o, l = good(o_parts, lse_parts)
        return np.asarray(o_parts, float).mean(axis=0), l

    return [no_max_shift, lse_without_shift, unnormalised_output, max_instead_of_logsumexp,
            reversed_weights, plain_average]


def _failed_merge_pins(monkeypatch, bad):
    import sys
    mod = sys.modules[__name__]
    monkeypatch.setattr(mod, "merge_lse_fp64", bad)
    failed = []
    pins = [lambda: test_merge_of_key_parts_is_the_full_attention([0, 17, 18, 33, 49, 50]),
            lambda: test_merge_of_key_parts_is_the_full_attention([0, 25, 50]),
            test_merge_invariants, test_merge_far_beyond_exp_range]
    for i, pin in enumerate(pins):
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed.append(i)
    return failed


def test_planted_mistakes_fail_a_pin(monkeypatch):
    """Each plausible slip in the merge (no max shift, the shift dropped from
    LSE, the output left unnormalised, max in place of log-sum-exp, reversed
    weights, a plain average of the parts) fails at least one pin above; the
    merge as written fails none."""
    assert _failed_merge_pins(monkeypatch, merge_lse_fp64) == []
    for bad in _merge_mutants():
        assert _failed_merge_pins(monkeypatch, bad), bad.__name__
