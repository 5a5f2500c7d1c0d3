"""Pins for the CPU oracle: it is checked against what the pages and the
mathematics fix, never against itself or the HIP path.

Sources: "3.6 Attention I -- the memory problem and FlashAttention
principles" (sections 3.6.4 recurrence, 3.6.5 worked example, 3.6.6 tile
loop and causal rule, 3.6.7 L = m + log l, 3.6.10 pitfalls, 3.6.11 exercise
2), and the one-query-block pseudocode of "A learning journey: CUDA, Triton,
Flash Attention".
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_fp64, attention_probs_fp64, brute_force_attention,
                    online_softmax_attention)
from exact_attention_fwd_amd.workloads import make_qkv, sample_rows, stress_inputs


def _row_problem(scores, values):
    """One query row whose scores are exactly ``scores`` (d = 1, scale 1)."""
    n = len(scores)
    q = np.zeros((1, 1, n, 1))
    q[0, 0, :, 0] = 1.0
    k = np.asarray(scores, dtype=np.float64).reshape(1, 1, n, 1)
    v = np.asarray(values, dtype=np.float64).reshape(1, 1, n, 1)
    return q, k, v


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example
def test_worked_example_full_softmax(golden_dir):
    g = _load(golden_dir, "worked_example_online_softmax.json")
    q, k, v = _row_problem(g["scores"], g["values"])
    o, lse, m, l = attention_fp64(q, k, v, 1.0, rows=[0], return_stats=True)
    full = g["full"]
    assert m[0, 0, 0] == full["m"]
    assert abs(l[0, 0, 0] - full["l"]) <= full["l_tol"]
    assert abs(o[0, 0, 0, 0] - full["O"]) <= full["O_tol"]
    assert abs(o[0, 0, 0, 0] * l[0, 0, 0] - full["numerator"]) <= full["numerator_tol"]
    probs = attention_probs_fp64(q, k, 1.0)[0, 0, 0]
    weights = probs * l[0, 0, 0]
    np.testing.assert_allclose(weights, full["weights"], atol=full["weights_tol"], rtol=0)
    np.testing.assert_allclose(weights * np.asarray(g["values"]), full["weighted_terms"],
                               atol=full["weighted_terms_tol"], rtol=0)
    # LSE = m + ln l, the statistic kept for the backward pass (3.6.7).
    assert lse[0, 0, 0] == pytest.approx(5 + math.log(l[0, 0, 0]), abs=1e-15)


def test_worked_example_online_two_blocks(golden_dir):
    g = _load(golden_dir, "worked_example_online_softmax.json")
    q, k, v = _row_problem(g["scores"], g["values"])
    ob = g["online_two_blocks"]
    out, lse, st = online_softmax_attention(q[0, 0, :1], k[0, 0], v[0, 0], 1.0,
                                            blocks=ob["blocks"], trace=True)
    s1, s2 = st
    e1, e2 = ob["after_block_1"], ob["after_block_2"]
    assert s1["m_tilde"][0] == e1["m_tilde"] and s1["m_new"][0] == e1["m_new"]
    assert s1["alpha"][0] == e1["alpha"]
    np.testing.assert_allclose(s1["p"][0], e1["p"], atol=e1["p_tol"], rtol=0)
    assert abs(s1["l"][0] - e1["l"]) <= e1["l_tol"]
    assert abs(s1["o"][0, 0] - e1["O"]) <= e1["O_tol"]
    assert s2["m_tilde"][0] == e2["m_tilde"] and s2["m_new"][0] == e2["m_new"]
    assert abs(s2["alpha"][0] - e2["alpha"]) <= e2["alpha_tol"]
    np.testing.assert_allclose(s2["p"][0], e2["p"], atol=e2["p_tol"], rtol=0)
    assert abs(s2["l"][0] - e2["l"]) <= e2["l_tol"]
    assert abs(s2["o"][0, 0] - e2["O"]) <= e2["O_tol"]
    assert abs(out[0, 0] - ob["O_final"]) <= ob["O_final_tol"]
    # The page: taking block 2 first gives the same result.
    out_r, lse_r = online_softmax_attention(q[0, 0, :1], k[0, 0], v[0, 0], 1.0,
                                            blocks=ob["blocks"], order=[1, 0])
    assert ob["reversed_order_same_result"]
    assert out_r[0, 0] == pytest.approx(out[0, 0], rel=1e-14)
    assert lse_r[0] == pytest.approx(lse[0], rel=1e-14)
    # and the full computation agrees with both
    o_full, lse_full = attention_fp64(q, k, v, 1.0, rows=[0])
    assert o_full[0, 0, 0, 0] == pytest.approx(out[0, 0], rel=1e-14)
    assert lse_full[0, 0, 0] == pytest.approx(lse[0], rel=1e-14)


def test_exercise2_constant_values(golden_dir):
    g = _load(golden_dir, "exercise2_constant_values.json")
    q, k, v = _row_problem(g["scores"], g["values"])
    out, lse, st = online_softmax_attention(q[0, 0, :1], k[0, 0], v[0, 0], 1.0,
                                            blocks=g["blocks"], trace=True)
    assert out[0, 0] == pytest.approx(g["O_final"], abs=1e-15)
    # closed form of this test's own: l = e^(0-4) + e^(2-4) + e^(4-4)
    l_closed = 1.0 + math.exp(-2.0) + math.exp(-4.0)
    assert st[-1]["l"][0] == pytest.approx(l_closed, rel=1e-15)
    assert lse[0] == pytest.approx(4.0 + math.log(l_closed), rel=1e-15)
    o_full, _ = attention_fp64(q, k, v, 1.0, rows=[0])
    assert o_full[0, 0, 0, 0] == pytest.approx(1.0, abs=1e-15)


# ------------------------------------------------------------------ closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_weights_when_scale_is_zero(causal):
    q, k, v = make_qkv(2, 2, 37, 8, seed=3)
    o, lse = attention_fp64(q, k, v, 0.0, causal=causal)
    v64 = v.astype(np.float64)
    n = q.shape[2]
    for i in range(n):
        vis = i + 1 if causal else n
        np.testing.assert_allclose(o[:, :, i], v64[:, :, :vis].mean(axis=2), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], math.log(vis), rtol=0, atol=1e-13)


def test_uniform_weights_when_q_is_zero():
    q, k, v = stress_inputs("zero_q", 1, 2, 19, 4)
    o, lse = attention_fp64(q, k, v, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(v.astype(np.float64).mean(axis=2, keepdims=True), o.shape),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(19), rtol=0, atol=1e-13)


def test_causal_row_zero_sees_only_key_zero():
    q, k, v = make_qkv(2, 3, 16, 8, seed=5)
    scale = 0.35
    o, lse = attention_fp64(q, k, v, scale, causal=True)
    sigma = float(np.float32(scale))
    for b in range(2):
        for h in range(3):
            assert np.array_equal(o[b, h, 0], v[b, h, 0].astype(np.float64))
            dot = math.fsum(float(x) * float(y) for x, y in zip(q[b, h, 0], k[b, h, 0]))
            assert lse[b, h, 0] == pytest.approx(sigma * dot, rel=1e-15, abs=1e-15)


def test_one_dominant_key_selects_its_value():
    q, k, v = make_qkv(1, 1, 24, 4, seed=7)
    q = q.astype(np.float64)
    k = k.astype(np.float64)
    q[..., :] = 0.0
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    j_star = 13
    k[0, 0, j_star, 0] = 50.0           # score 50 against 0 for all others
    o, lse = attention_fp64(q, k, v, 1.0)
    bound = 23 * math.exp(-50.0) * np.abs(v).max() * 2
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, j_star].astype(np.float64), (24, 4)),
                               rtol=0, atol=bound)
    np.testing.assert_allclose(lse, 50.0 + math.log1p(23 * math.exp(-50.0)), rtol=1e-15)


def test_permutation_equivariance():
    q, k, v = make_qkv(1, 2, 29, 8, seed=11)
    rng = np.random.default_rng(0)
    o, lse = attention_fp64(q, k, v, 0.3)
    pk = rng.permutation(29)
    o2, lse2 = attention_fp64(q, k[:, :, pk], v[:, :, pk], 0.3)      # keys with values
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)
    pq = rng.permutation(29)
    o3, lse3 = attention_fp64(q[:, :, pq], k, v, 0.3)                 # queries
    np.testing.assert_allclose(o3, o[:, :, pq], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse3, lse[:, :, pq], rtol=1e-14)
    # keys permuted without their values must change the result
    o4, _ = attention_fp64(q, k[:, :, pk], v, 0.3)
    assert np.abs(o4 - o).max() > 1e-3


def test_head_independence():
    q, k, v = make_qkv(2, 3, 12, 4, seed=13)
    o, lse = attention_fp64(q, k, v, 0.5)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[1, 2] *= -1
    k2[1, 2] = k2[1, 2, ::-1]
    v2[1, 2] += 1
    o2, lse2 = attention_fp64(q2, k2, v2, 0.5)
    mask = np.ones((2, 3), bool)
    mask[1, 2] = False
    assert np.array_equal(o2[mask], o[mask]) and np.array_equal(lse2[mask], lse[mask])
    assert not np.allclose(o2[1, 2], o[1, 2])


def test_zero_padding_head_dim_leaves_scores_unchanged():
    q, k, v = make_qkv(1, 2, 17, 3, seed=17)
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (5,), x.dtype)], axis=-1)
    for causal in (False, True):
        o, lse = attention_fp64(q, k, v, 0.7, causal=causal)
        op, lsep = attention_fp64(pad(q), pad(k), pad(v), 0.7, causal=causal)
        np.testing.assert_allclose(op[..., :3], o, rtol=1e-14, atol=1e-15)
        assert np.all(op[..., 3:] == 0)
        np.testing.assert_allclose(lsep, lse, rtol=1e-15)


def test_negative_scale_equals_flipped_queries():
    q, k, v = make_qkv(1, 1, 21, 8, seed=19)
    o, lse = attention_fp64(q, k, v, -0.25, causal=True)
    o2, lse2 = attention_fp64(-q, k, v, 0.25, causal=True)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=1e-15)


def test_scale_is_the_fp32_value():
    q, k, v = make_qkv(1, 1, 8, 128, seed=23)
    s64 = 1.0 / math.sqrt(128.0)
    s32 = float(np.float32(s64))
    assert s32 != s64
    _, lse_a = attention_fp64(q, k, v, s64)
    _, lse_b = attention_fp64(q, k, v, s32)
    assert np.array_equal(lse_a, lse_b)
    # ... and it is not silently the fp64 value: compare with a direct sum
    dot = math.fsum(float(x) * float(y) for x, y in zip(q[0, 0, 0], k[0, 0, 0]))
    _, lse_c, m, _ = attention_fp64(q, k, v, s64, rows=[0], return_stats=True)
    s_all = [s32 * math.fsum(float(x) * float(y) for x, y in zip(q[0, 0, 0], k[0, 0, j])) for j in range(8)]
    assert m[0, 0, 0] == pytest.approx(max(s_all), rel=1e-15)
    assert dot != 0


# -------------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one_and_masked_entries_vanish(causal):
    q, k, _ = make_qkv(2, 2, 33, 16, seed=29)
    p = attention_probs_fp64(q, k, 0.25, causal=causal)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)
    if causal:
        iu = np.triu_indices(33, k=1)
        assert np.all(p[:, :, iu[0], iu[1]] == 0)
        assert np.all(p[:, :, np.arange(33), np.arange(33)] > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_output_in_convex_hull_and_lse_bounds(causal):
    q, k, v = make_qkv(1, 3, 40, 8, seed=31)
    o, lse, m, l = attention_fp64(q, k, v, 0.4, causal=causal, return_stats=True)
    v64 = v.astype(np.float64)
    for i in range(40):
        vis = slice(0, i + 1) if causal else slice(0, 40)
        lo = v64[:, :, vis].min(axis=2)
        hi = v64[:, :, vis].max(axis=2)
        assert np.all(o[:, :, i] >= lo - 1e-13) and np.all(o[:, :, i] <= hi + 1e-13)
        n_vis = (i + 1) if causal else 40
        assert np.all(lse[:, :, i] >= m[:, :, i] - 1e-15)
        assert np.all(lse[:, :, i] <= m[:, :, i] + math.log(n_vis) + 1e-13)
    assert np.all(l >= 1.0 - 1e-15)


# --------------------------------------------------- online variant vs the oracle
@pytest.mark.parametrize("causal", [False, True])
def test_online_variant_matches_for_any_block_size_and_order(causal):
    q, k, v = make_qkv(1, 1, 45, 8, seed=37)
    o, lse = attention_fp64(q, k, v, 0.5, causal=causal)
    rng = np.random.default_rng(1)
    for bs in [1, 2, 3, 7, 16, 44, 45, 64]:
        nblk = -(-45 // bs)
        for trial in range(3):
            order = rng.permutation(nblk) if trial else None
            oo, ll = online_softmax_attention(q[0, 0], k[0, 0], v[0, 0], 0.5, causal=causal,
                                              block_size=bs, order=order)
            np.testing.assert_allclose(oo, o[0, 0], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(ll, lse[0, 0], rtol=1e-12)
    # uneven random partitions, processed in random order
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 45), size=6, replace=False))
        blocks = np.split(rng.permutation(45) if not causal else np.arange(45), cuts)
        order = rng.permutation(len(blocks))
        oo, ll = online_softmax_attention(q[0, 0], k[0, 0], v[0, 0], 0.5, causal=causal,
                                          blocks=blocks, order=order)
        np.testing.assert_allclose(oo, o[0, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ll, lse[0, 0], rtol=1e-12)


@pytest.mark.parametrize("kind", ["rising", "falling"])
def test_online_variant_on_moving_maximum(kind):
    q, k, v = stress_inputs(kind, 1, 1, 64, 8)
    o, lse = attention_fp64(q, k, v, 1.0)
    oo, ll, st = online_softmax_attention(q[0, 0], k[0, 0], v[0, 0], 1.0, block_size=8, trace=True)
    np.testing.assert_allclose(oo, o[0, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ll, lse[0, 0], rtol=1e-12)
    alphas = np.array([s["alpha"] for s in st[1:]])
    assert np.all(alphas <= 1.0)                  # alpha <= 1 (3.6.4)
    if kind == "rising":
        assert np.all(alphas < 1.0)               # the max grows on every block
    else:
        assert np.all(alphas == 1.0)              # the max never grows after block 0


def test_negative_controls_fail_by_far():
    """The 3.6.10 pitfalls, planted in the oracle's online variant."""
    q, k, v = stress_inputs("rising", 1, 1, 64, 8)
    o, lse = attention_fp64(q, k, v, 1.0)
    args = (q[0, 0], k[0, 0], v[0, 0], 1.0)
    for mode in ("l_only", "o_only"):
        oo, _ = online_softmax_attention(*args, block_size=8, rescale=mode)
        assert np.abs(oo - o[0, 0]).max() > 0.1, mode
    # without the max shift the exponentials overflow at scores ~ 1000
    qb, kb, vb = stress_inputs("large", 1, 1, 32, 64)
    qb = qb.astype(np.float64) * 8
    o_ok, lse_ok = online_softmax_attention(qb[0, 0], kb[0, 0], vb[0, 0], 1.0, block_size=8)
    assert np.all(np.isfinite(o_ok)) and np.all(np.isfinite(lse_ok))
    o_bad, _ = online_softmax_attention(qb[0, 0], kb[0, 0], vb[0, 0], 1.0, block_size=8, max_shift=False)
    assert not np.all(np.isfinite(o_bad))


# ------------------------------------------- independent implementations to agree
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_float64(causal):
    torch = pytest.importorskip("torch")
    q, k, v = make_qkv(1, 2, 256, 64, seed=0)
    o, lse = attention_fp64(q, k, v, 0.125, causal=causal)
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.125)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)
    s = 0.125 * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(256, 256, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 17])
@pytest.mark.parametrize("d", [1, 2, 4])
def test_against_pure_python_brute_force(n, d, causal):
    B, H = (2, 1) if n % 2 else (1, 2)
    q, k, v = make_qkv(B, H, n, d, sigma=1.5, seed=100 + n * 10 + d)
    o, lse = attention_fp64(q, k, v, 0.6, causal=causal)
    ob, lb = brute_force_attention(q, k, v, 0.6, causal=causal)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-14)


def test_sampled_rows_equal_full_rows():
    q, k, v = make_qkv(2, 2, 700, 16, seed=41)
    o, lse = attention_fp64(q, k, v, 0.25, causal=True)
    rows = np.stack([np.stack([sample_rows(700, b, h, 64) for h in range(2)]) for b in range(2)])
    o_s, lse_s = attention_fp64(q, k, v, 0.25, causal=True, rows=rows, row_block=10)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(o_s[b, h], o[b, h, rows[b, h]], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse_s[b, h], lse[b, h, rows[b, h]], rtol=1e-14)


def test_threads_do_not_change_results():
    q, k, v = make_qkv(2, 4, 130, 8, seed=43)
    a = attention_fp64(q, k, v, 0.3, causal=True, threads=1)
    b = attention_fp64(q, k, v, 0.3, causal=True, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sample_rows_contract():
    r = sample_rows(65536, 0, 3)
    assert len(r) == 512 and r[0] == 0 and r[-1] == 65535 and len(np.unique(r)) == 512
    assert np.array_equal(r, sample_rows(65536, 0, 3))
    assert not np.array_equal(r, sample_rows(65536, 0, 4))
    assert np.array_equal(sample_rows(300, 1, 1), np.arange(300))


def test_large_scores_stay_finite():
    """Scores near 1000 overflow exp unless the row max is subtracted (3.6.10)."""
    q, k, v = stress_inputs("large", 1, 2, 48, 64)
    q = q.astype(np.float64) * 8
    o, lse = attention_fp64(q, k, v, 1.0, causal=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.abs(lse).max() > 800
    p = attention_probs_fp64(q, k, 1.0, causal=True)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-12)


# ------------------------------------------------ planted mistakes fail a pin
def _mutant_rows():
    """Plausible slips in the oracle's per-block step (each a replacement for
    oracle.attention._attention_rows, same signature and returns)."""
    import oracle.attention as oa

    def scores(q_rows, row_ids, k, sigma, causal, shift=0):
        s = sigma * (q_rows @ k.T)
        if causal:
            keys = np.arange(k.shape[0])
            s[keys[None, :] > row_ids[:, None] + shift] = -np.inf
        return s

    def finish(s, v, weights=None):
        m = s.max(axis=1)
        p = np.exp(s - m[:, None]) if weights is None else weights(s, m)
        l = p.sum(axis=1)
        return (p @ v) / l[:, None], m + np.log(l), m, l

    def causal_off_by_one(q_rows, row_ids, k, v, sigma, causal):
        return finish(scores(q_rows, row_ids, k, sigma, causal, shift=1), v)

    def wrong_operand(q_rows, row_ids, k, v, sigma, causal):
        return finish(scores(q_rows, row_ids, k, sigma, causal), k)

    def no_max_shift(q_rows, row_ids, k, v, sigma, causal):
        s = scores(q_rows, row_ids, k, sigma, causal)
        p = np.exp(s)
        l = p.sum(axis=1)
        return (p @ v) / l[:, None], np.log(l), np.zeros(len(l)), l

    def lse_without_max(q_rows, row_ids, k, v, sigma, causal):
        o, _, m, l = finish(scores(q_rows, row_ids, k, sigma, causal), v)
        return o, np.log(l), m, l

    def no_normaliser(q_rows, row_ids, k, v, sigma, causal):
        o, lse, m, l = finish(scores(q_rows, row_ids, k, sigma, causal), v)
        return o * l[:, None], lse, m, l

    def biased_sum(q_rows, row_ids, k, v, sigma, causal):
        s = scores(q_rows, row_ids, k, sigma, causal)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1) * (1 + 1e-6)
        return (p @ v) / l[:, None], m + np.log(l), m, l

    def missing_scale(q_rows, row_ids, k, v, sigma, causal):
        return finish(scores(q_rows, row_ids, k, 1.0, causal), v)

    def reversed_weights(q_rows, row_ids, k, v, sigma, causal):
        def w(s, m):
            p = np.exp(np.where(np.isfinite(s), m[:, None] - s, -np.inf))
            return p
        return finish(scores(q_rows, row_ids, k, sigma, causal), v, w)

    return oa, [causal_off_by_one, wrong_operand, no_max_shift, lse_without_max,
                no_normaliser, biased_sum, missing_scale, reversed_weights]


def _failed_pins(golden_dir):
    """Run a set of the pins above; return the names of those that fail."""
    pins = [
        ("worked example", lambda: test_worked_example_full_softmax(golden_dir)),
        ("causal row 0", test_causal_row_zero_sees_only_key_zero),
        ("fp32 scale", test_scale_is_the_fp32_value),
        ("large scores", test_large_scores_stay_finite),
        ("brute force", lambda: [test_against_pure_python_brute_force(5, 2, c) for c in (False, True)]),
        ("convex hull", lambda: [test_output_in_convex_hull_and_lse_bounds(c) for c in (False, True)]),
    ]
    failed = []
    for name, pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    return failed


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_planted_mistakes_fail_a_pin(golden_dir, monkeypatch):
    """Each plausible slip in the oracle's block step -- causal off by one,
    the wrong operand in the second product, no max shift, the LSE without
    m, no normalisation, a biased row sum, the scale left out, weights
    reversed -- and the scale taken in fp64 instead of the fp32 value fail
    at least one pin; the unmodified oracle fails none."""
    assert _failed_pins(golden_dir) == []
    oa, mutants = _mutant_rows()
    good = oa._attention_rows
    for bad in mutants:
        monkeypatch.setattr(oa, "_attention_rows", bad)
        failed = _failed_pins(golden_dir)
        monkeypatch.setattr(oa, "_attention_rows", good)
        assert failed, bad.__name__
    good_sigma = oa._sigma
    monkeypatch.setattr(oa, "_sigma", lambda scale: float(scale))
    failed = _failed_pins(golden_dir)
    monkeypatch.setattr(oa, "_sigma", good_sigma)
    assert failed, "fp64 scale"
