"""GPU parity: the HIP attention forward against the float64 CPU oracle, on the
same seeded inputs, through the C ABI (python binding -> libfa2.so).

Workloads: the five configurations of the pages' shapes (tiny, [4,32,2048,64]
non-causal and causal, [2,16,16384,128], [1,16,65536,128] non-causal and
causal) plus [4,32,2048,128] and the head-dim cases [4,32,2048,32],
[4,32,2048,96], [4,16,2048,256] (also causal); large ones are checked on 512 seeded query rows
per (batch, head) and, for every element, on properties that hold at any
size (finiteness, closed forms).  Edge cases: the pages' worked example
embedded in d = 64, odd N (tails) at every head dim, stress inputs that move the running max,
scale 0 / negative, determinism, NaN-poisoned and guard-banded outputs.
"""
import functools
import math

import numpy as np
import pytest

from exact_attention_fwd_amd.workloads import WORKLOADS, make_qkv, sample_rows, stress_inputs
from oracle import attention_fp64
from parity import diff, run_gpu, say

pytestmark = pytest.mark.gpu

HEAD_DIMS = [32, 64, 96, 128, 256]

torch = pytest.importorskip("torch")


@functools.lru_cache(maxsize=2)
def inputs(B, H, N, d, sigma, seed):
    return make_qkv(B, H, N, d, sigma, seed)


def check(name, q, k, v, scale, causal, rows=None):
    o, l = run_gpu(q, k, v, scale, causal)
    assert np.all(np.isfinite(o.astype(np.float32))) and np.all(np.isfinite(l)), name
    if rows is None:
        o_ref, l_ref = attention_fp64(q, k, v, scale, causal=causal)
        og, lg = o, l
    else:
        o_ref, l_ref = attention_fp64(q, k, v, scale, causal=causal, rows=rows)
        bi = np.arange(q.shape[0])[:, None, None]
        hi = np.arange(q.shape[1])[None, :, None]
        og, lg = o[bi, hi, rows], l[bi, hi, rows]
    dd = diff(og, lg, o_ref, l_ref)
    say(f"[parity] {name}: {dd}")
    assert dd.ok(), f"{name}: {dd}"
    return o, l


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("name", ["tiny", "ref", "ref_causal"])
def test_workload_full(name):
    w = WORKLOADS[name]
    q, k, v = inputs(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    check(name, q, k, v, w.scale, w.causal)


def test_tiny_causal():
    w = WORKLOADS["tiny"]
    q, k, v = inputs(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    check("tiny_causal", q, k, v, w.scale, True)


@pytest.mark.parametrize("name", ["ref_d128", "hd128_16k", "long_64k", "long_64k_causal",
                                  "hd32", "hd96", "hd256", "hd256_causal"])
def test_workload_sampled(name):
    w = WORKLOADS[name]
    q, k, v = inputs(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    rows = np.stack([np.stack([sample_rows(w.N, b, h, w.sampled_rows) for h in range(w.H)])
                     for b in range(w.B)])
    check(name, q, k, v, w.scale, w.causal, rows=rows)


# ------------------------------------------------ the pages' worked examples
def _embed(scores, values, d=64):
    """One head whose every query row has exactly the given scores (scale 1)."""
    n = len(scores)
    q = np.zeros((1, 1, n, d), np.float16)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[..., 0] = 1
    k[0, 0, :, 0] = scores
    v[0, 0, :, 0] = values
    return q, k, v


def test_worked_example_in_d64():
    # "Attention I", 3.6.5: scores [1,3,2,5], values [10,20,30,40] -> 36.88,
    # l = 1.2034.  fp16 rounds 36.880566 to 36.875 (far from the midpoint).
    q, k, v = _embed([1, 3, 2, 5], [10, 20, 30, 40])
    o, l = run_gpu(q, k, v, 1.0, False)
    assert np.all(o[..., 0] == np.float16(36.875)), o[..., 0]
    assert np.all(o[..., 1:] == 0)
    lse = 5.0 + math.log(1 + math.exp(-4) + math.exp(-2) + math.exp(-3))
    np.testing.assert_allclose(l, lse, rtol=1e-6)
    # causal: row 0 sees only key 0 -> exactly v_0 and LSE = s_00 = 1
    o, l = run_gpu(q, k, v, 1.0, True)
    assert o[0, 0, 0, 0] == 10 and l[0, 0, 0] == pytest.approx(1.0, abs=1e-6)


def test_exercise2_constant_values_in_d64():
    # "Attention I", 3.6.11 exercise 2: scores [0,2,4], all values 1 -> O = 1.
    q, k, v = _embed([0, 2, 4], [1, 1, 1])
    o, l = run_gpu(q, k, v, 1.0, False)
    assert np.all(np.abs(o[..., 0].astype(np.float64) - 1.0) <= 2.0 ** -10)
    np.testing.assert_allclose(l, 4 + math.log(1 + math.exp(-2) + math.exp(-4)), rtol=1e-6)


# -------------------------------------------------------------- tails, odd N
@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 4, 17, 63, 65, 129, 1000])
def test_odd_lengths(n, d, causal):
    q, k, v = make_qkv(1, 2, n, d, 1.0, seed=n)
    check(f"N={n} d={d} causal={causal}", q, k, v, d ** -0.5, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [8192 + 37, 8192 + 193])
def test_long_ragged_d128(n, causal):
    """From N = 8192 the d = 128 kernel keeps a ring of four K/V tiles per
    tensor (one barrier per two tiles); ragged ends at both tile parities."""
    q, k, v = make_qkv(1, 2, n, 128, 1.0, seed=n)
    check(f"N={n} d=128 causal={causal}", q, k, v, 128 ** -0.5, causal)


@pytest.mark.parametrize("n,kind", [(2048, "random"), (4096 + 37, "random"), (2048, "rising"),
                                    (4096 + 37, "falling")])
def test_causal_d64_long_rows(n, kind):
    """Causal d = 64 from N = 2048 on grids of >= 256 such workgroups runs
    256-query workgroups with a ring of four K/V tiles (shorter rows: 128),
    where waves whose queries all precede the last key tile skip its
    softmax.  Ragged end included, and rows whose max rises with every key
    tile (rising) or sits in the first (falling); 256 sampled rows per head,
    the last rows among them."""
    B, H = 1, 40
    if kind == "random":
        q, k, v = make_qkv(B, H, n, 64, 1.0, seed=n + 1)
    else:
        q, k, v = stress_inputs(kind, B, H, n, 64, seed=n + 1)
    rows = np.stack([np.stack([np.unique(np.concatenate([sample_rows(n, b, h, 256),
                                                         np.arange(n - 300, n)]))[-256:]
                               if h % 2 else sample_rows(n, b, h, 256) for h in range(H)])
                     for b in range(B)])
    check(f"causal d=64 N={n} {kind}", q, k, v, 1.0 if kind != "random" else 0.125, True, rows=rows)


@pytest.mark.parametrize("B,H,N,causal", [(1, 4, 2048, True), (1, 32, 2048, True), (1, 8, 16384 + 37, False)])
def test_d64_launch_shapes(B, H, N, causal):
    """Each d = 64 launch choice at full size: causal rows of 2048 on a grid
    too small for the 256-query groups (B*H = 4: 128-query groups, ring of
    two), causal exactly at the boundary where the 256-query groups start
    (B*H = 32: 256 of them), and long non-causal rows with a ragged end
    (256-query groups, ring of four, 257 key tiles); 256 sampled rows per
    head, the last rows among them."""
    q, k, v = make_qkv(B, H, N, 64, 1.0, seed=N + H + B)
    tail = np.arange(N - 64, N)
    rows = np.stack([np.stack([np.sort(np.concatenate([np.setdiff1d(sample_rows(N, b, h, 256), tail)[:192],
                                                       tail])) for h in range(H)]) for b in range(B)])
    check(f"[{B},{H},{N},64] causal={causal}", q, k, v, 0.125, causal, rows=rows)


@pytest.mark.parametrize("kind", ["rising", "falling"])
def test_long_moving_max_d128(kind):
    q, k, v = stress_inputs(kind, 1, 1, 8192 + 5, 128, seed=4)
    for causal in (False, True):
        check(f"stress {kind} N=8197 d=128 causal={causal}", q, k, v, 1.0, causal)


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_batch_heads_and_ragged_tail_together(d):
    q, k, v = make_qkv(3, 5, 300, d, 1.0, seed=7)
    for causal in (False, True):
        check(f"[3,5,300,{d}] causal={causal}", q, k, v, d ** -0.5, causal)


@pytest.mark.parametrize("kind,B,H,N,scale", [
    ("random", 2, 160, 256, 0.125), ("random", 1, 300, 512, -0.125), ("random", 4, 72, 1024, 0.125),
    ("rising", 2, 160, 256, 1.0), ("falling", 1, 300, 512, 1.0), ("large", 2, 160, 256, 0.125)])
def test_many_units_per_workgroup(kind, B, H, N, scale):
    """Grids of 320 to 1152 (Q tile, head) units, more than the chip runs at
    once, with the row max moving (rising keys), fixed in the first tile
    (falling), far beyond exp's range (large) and a negative scale."""
    if kind == "random":
        q, k, v = make_qkv(B, H, N, 64, 1.0, seed=N + H)
    else:
        q, k, v = stress_inputs(kind, B, H, N, 64, seed=N + H)
    check(f"{kind} [{B},{H},{N},64] scale={scale}", q, k, v, scale, False)


# ----------------------------------------------------------- stress inputs
@pytest.mark.parametrize("kind", ["rising", "falling", "large", "const_v", "zero_q"])
@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_stress(kind, d, causal):
    q, k, v = stress_inputs(kind, 1, 2, 333, d, seed=3)
    check(f"stress {kind} d={d} causal={causal}", q, k, v, 1.0 if kind in ("rising", "falling") else d ** -0.5,
          causal)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3, 1e-3])
def test_scale_values(scale):
    q, k, v = make_qkv(1, 2, 200, 64, 1.0, seed=11)
    for causal in (False, True):
        check(f"scale={scale} causal={causal}", q, k, v, scale, causal)


@pytest.mark.parametrize("scale", [1000.0, -1000.0])
def test_sharp_softmax_is_a_hard_argmax(scale):
    """|scale| = 1000 at d = 64 (scaled scores up to about 6e4, inside the
    precision range the header states): the softmax is a hard argmax for
    every row whose two best scores are apart by more than 30 / (|scale|
    log2 e) -- the runner-up weight is then below 2^-30 -- so O is the V
    row of the best key to fp16 rounding, and LSE is scale times that
    key's score up to the fp32 rounding of the score."""
    q, k, v = make_qkv(1, 2, 200, 64, 1.0, seed=11)
    for causal in (False, True):
        o, l = run_gpu(q, k, v, scale, causal)
        assert np.all(np.isfinite(o.astype(np.float32))) and np.all(np.isfinite(l))
        q64, k64 = q.astype(np.float64), k.astype(np.float64)
        s = scale * np.einsum("bhid,bhjd->bhij", q64, k64)
        mag = abs(scale) * np.einsum("bhid,bhjd->bhij", np.abs(q64), np.abs(k64))
        if causal:
            s = np.where(np.tril(np.ones(s.shape[-2:], bool)), s, -np.inf)
        best = np.argmax(s, axis=-1)
        top2 = np.sort(s, axis=-1)[..., -2:]
        slack = 64 * 2.0 ** -24 * np.take_along_axis(mag, best[..., None], -1)[..., 0]
        clear = (top2[..., 1] - top2[..., 0]) * math.log2(math.e) > 30 + 4 * slack
        say(f"[parity] scale={scale:g} causal={causal}: {clear.mean():.3f} of the rows checked")
        assert clear.mean() > 0.9
        want_o = v[np.arange(1)[:, None, None], np.arange(2)[None, :, None], best].astype(np.float32)
        err_o = np.abs(o.astype(np.float32) - want_o)
        # other weights sum to at most 200 * 2^-30 of the best one
        assert np.all(err_o[clear] <= 2.0 ** -10 * np.abs(want_o[clear]) + 4e-6)
        want_l = top2[..., 1]
        err_l = np.abs(l.astype(np.float64) - want_l)
        assert np.all(err_l[clear] <= slack[clear] + 4 * 2.0 ** -24 * np.abs(want_l[clear]) + 1e-6)


# ----------------------------------------- full-size properties, every element
@pytest.mark.parametrize("causal", [False, True])
def test_full_size_closed_forms(causal):
    """[1,16,65536,128]: with Q = 0 every weight is equal, so LSE is ln of the
    visible-key count for every row; with constant V every output is that V."""
    w = WORKLOADS["long_64k"]
    _, k, v = inputs(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    q0 = np.zeros_like(k)
    o, l = run_gpu(q0, k, v, w.scale, causal)
    n_vis = np.arange(1, w.N + 1) if causal else np.full(w.N, w.N)
    np.testing.assert_allclose(l, np.broadcast_to(np.log(n_vis), l.shape), rtol=2e-6)
    if causal:
        assert np.array_equal(o[:, :, 0], v[:, :, 0])   # row 0 sees key 0 only
    vc = np.broadcast_to(v[:, :, :1], v.shape).copy()
    qq, _, _ = inputs(w.B, w.H, w.N, w.d, w.sigma, w.seed)
    o, l = run_gpu(qq, k, vc, w.scale, causal)
    err = np.abs(o.astype(np.float32) - vc.astype(np.float32))
    say(f"[parity] full-size constant V causal={causal}: max|O-v0|={err.max():.3e}")
    assert err.max() <= 2 ** -11 * np.abs(vc).astype(np.float32).max() * 2
    assert np.all(np.isfinite(l))


# ------------------------------------------------------ run-level guarantees
def test_deterministic_and_overwrites_poisoned_outputs():
    q, k, v = make_qkv(2, 4, 777, 128, 1.0, seed=5)
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    import exact_attention_fwd_amd as fa2
    for causal in (False, True):
        out = torch.full_like(tq, float("nan"))
        lse = torch.full((2, 4, 777), float("nan"), device="cuda")
        o1, l1 = fa2.fwd(tq, tk, tv, causal=causal, out=out, lse=lse)
        o2, l2 = fa2.fwd(tq, tk, tv, causal=causal)
        torch.cuda.synchronize()
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_guard_bands_untouched():
    import exact_attention_fwd_amd as fa2
    B, H, N, d, guard = 1, 3, 257, 64, 512
    q, k, v = make_qkv(B, H, N, d, 1.0, seed=9)
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    n_o, n_l = B * H * N * d, B * H * N
    o_buf = torch.full((n_o + 2 * guard,), 7.0, dtype=torch.float16, device="cuda")
    l_buf = torch.full((n_l + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    out = o_buf[guard:guard + n_o].view(B, H, N, d)
    lse = l_buf[guard:guard + n_l].view(B, H, N)
    fa2.fwd(tq, tk, tv, out=out, lse=lse, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o_buf[:guard] == 7) and torch.all(o_buf[guard + n_o:] == 7)
    assert torch.all(l_buf[:guard] == 7) and torch.all(l_buf[guard + n_l:] == 7)
    o_ref, l_ref = attention_fp64(q, k, v, d ** -0.5, causal=True)
    dd = diff(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)
    assert dd.ok(), str(dd)


def test_runs_on_the_callers_stream():
    import exact_attention_fwd_amd as fa2
    q, k, v = make_qkv(1, 2, 512, 64, 1.0, seed=13)
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    ref_o, ref_l = fa2.fwd(tq, tk, tv)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = fa2.fwd(tq, tk, tv)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jump", [3.0, 20.0])
def test_row_max_jumps_mid_sequence(d, causal, jump):
    """Scores ~0 except one key per row block far into the sequence whose score
    jumps by `jump` (natural units).  A jump of 20 (29 in log2 units) forces a
    rescale in the middle of the key loop; a jump of 3 (4.3 in log2 units) is
    absorbed without one.  Both must give the same softmax as the oracle."""
    n = 2048
    q, k, v = make_qkv(1, 2, n, d, 1.0, seed=17)
    q = (q.astype(np.float32) * 0.05).astype(np.float16)
    q[..., 0] = 1.0
    k = (k.astype(np.float32) * 0.05).astype(np.float16)
    k[..., 0] = 0.0
    k[:, :, 1500, 0] = jump
    k[:, :, 700, 0] = jump / 2
    check(f"jump={jump} d={d} causal={causal}", q, k, v, 1.0, causal)
