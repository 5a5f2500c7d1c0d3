"""Plain float64 CPU gradients of softmax attention: the oracle for the
backward kernels.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code may
import or call anything here.

What is differentiated.  The forward is the oracle's ``attention_fp64``: per
(batch, head), S = sigma Q K^T with future keys masked when causal, P the
row-wise softmax of S, O = P V ("3.6 Attention I -- the memory problem and
FlashAttention principles", 3.6.2 and 3.6.6).  Given an upstream gradient dO
of O, the gradients of the scalar <dO, O> with respect to Q, K and V are
returned.  The pages ask for exactly these three (3.6.7 of that chapter: the
backward recomputes S and P block by block from the row statistics the
forward stored; "A learning journey: CUDA, Triton, Flash Attention", the
closing list of exercises: derive dQ, dK, dV by hand) but print no formula,
so this module is the chain rule written out:

    dV = P^T dO                                   (O = P V, linear in V)
    dP = dO V^T                                   (linear in P)
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)       (Jacobian of a row softmax)
    dQ = sigma dS K,   dK = sigma dS^T Q          (S = sigma Q K^T)

Masked entries have P_ij = 0 and so dS_ij = 0.  The row term
sum_k P_ik dP_ik equals dO_i . O_i; it is returned as ``delta``.

Readings taken where the pages are silent: the loss is
<dO, O> (dO is the upstream gradient, any values); the scale is the fp32
value the kernel receives, widened exactly, as in the forward oracle; the
gradients are returned in float64, not rounded.

Every row of P is independent, so the rows are processed in blocks: dQ of a
block needs only that block, dK and dV sum the blocks' contributions.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import _masked_scores, _sigma, _stable_softmax_parts, oracle_threads

__all__ = ["attention_bwd_fp64", "attention_bwd_error_scale", "attention_bwd_error_std"]

# Absolute rounding error of an fp16 subnormal (2^-25) in units of the
# relative one (u = 2^-11).
_SUBNORMAL = 2.0 ** -14
# fp32 rounding (2^-24) in units of the fp16 one (2^-11).
_FP32_IN_U16 = 2.0 ** -13


def _bwd_rows(q_rows, row_ids, k, v, do_rows, sigma, causal):
    """Gradient contributions of a block of query rows of one (batch, head).

    Returns dQ rows [R, d], the rows' contributions to dK and dV [N, d], and
    delta [R] = sum_k P_ik dP_ik.  The forward steps are [Attn-I] 3.6.2 /
    3.6.4 / 3.6.6 (the same helpers as the forward oracle); the rest is the
    chain rule in the module docstring.
    """
    s = _masked_scores(q_rows, row_ids, k, sigma, causal)
    _, e, l = _stable_softmax_parts(s)
    p = e / l[:, None]                      # softmax rows; masked entries are 0
    dp = do_rows @ v.T                      # dL/dP
    delta = (p * dp).sum(axis=1)            # sum_k P_ik dP_ik
    ds = p * (dp - delta[:, None])          # dL/dS
    dq = sigma * (ds @ k)
    dk = sigma * (ds.T @ q_rows)
    dv = p.T @ do_rows
    return dq, dk, dv, delta


def attention_bwd_fp64(q, k, v, do, scale, causal=False, threads=None, row_block=None):
    """dQ, dK, dV of <dO, softmax(scale Q K^T) V> in float64, and delta.

    Arguments
      q, k, v, do : arrays [B, H, N, d] (fp16 inputs are widened exactly).
      scale  : the softmax scale, used as the fp32 value the kernel receives.
      causal : mask key j for query i when j > i.
      threads : worker threads over (b, h); BLAS is held to one thread each.
      row_block : query rows per materialised block (memory bound).

    Returns dq, dk, dv [B, H, N, d] and delta [B, H, N], all float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    if q.ndim != 4 or not (q.shape == k.shape == v.shape == do.shape):
        raise ValueError("q, k, v, do must share one shape [B, H, N, d]")
    B, H, N, d = q.shape
    sigma = _sigma(scale)
    if row_block is None:
        row_block = max(1, (1 << 21) // max(N, 1))  # ~16 MiB per fp64 block matrix
    dq = np.empty((B, H, N, d), dtype=np.float64)
    dk = np.empty((B, H, N, d), dtype=np.float64)
    dv = np.empty((B, H, N, d), dtype=np.float64)
    delta = np.empty((B, H, N), dtype=np.float64)

    def one_head(bh):
        b, h = divmod(bh, H)
        qh = q[b, h].astype(np.float64)
        kh = k[b, h].astype(np.float64)
        vh = v[b, h].astype(np.float64)
        doh = do[b, h].astype(np.float64)
        dk_acc = np.zeros((N, d))
        dv_acc = np.zeros((N, d))
        for r0 in range(0, N, row_block):
            ids = np.arange(r0, min(r0 + row_block, N))
            g_q, g_k, g_v, dl = _bwd_rows(qh[ids], ids, kh, vh, doh[ids], sigma, causal)
            dq[b, h, ids] = g_q
            delta[b, h, ids] = dl
            dk_acc += g_k
            dv_acc += g_v
        dk[b, h] = dk_acc
        dv[b, h] = dv_acc

    nthreads = threads or oracle_threads()
    if nthreads > 1 and B * H > 1:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=nthreads) as ex:
                list(ex.map(one_head, range(B * H)))
    else:
        for bh in range(B * H):
            one_head(bh)
    return dq, dk, dv, delta


def attention_bwd_error_scale(q, k, v, do, scale, causal=False, threads=None, row_block=None):
    """Per-element error scales E of dQ, dK, dV and delta, float64.

    Not part of what the kernels compute: the scale that a tolerance on
    their result is measured in.  A sum of products whose factors carry a
    relative error u (here u = 2^-11, fp16 rounding) is off by at most
    about u * sum |a| |b| -- the standard forward-error bound of a dot
    product.  Rounding to fp16 with gradual underflow gives
    fl(x) = x (1 + e) + a with |e| <= u and |a| <= 2^-25 (half the subnormal
    spacing), so a rounded factor x contributes u |x| + 2^-25, i.e.
    u (|x| + 2^-14 M) with M the visibility mask.  The gradients' factors
    that are rounded to fp16 on the way (P, dS), and the error of delta
    (taken from the fp16 O), give

        E_dV    = (|P| + t M)^T |dO|
        E_dQ    = |sigma| ((|dS| + t M) |K| + Dabs_i (|P| |K|))
        E_dK    = |sigma| ((|dS| + t M)^T |Q| + (|P| Dabs)^T |Q|)
        E_delta = Dabs_i = sum_c |dO_ic| |O_ic|,          t = 2^-14,

    where the Dabs terms bound how an error u * Dabs_i in delta_i moves
    dS_ij = P_ij (dP_ij - delta_i).  Where the gradient is a small
    difference of large terms (Q and K sharing a large component, or a
    constant V) E is much larger than |G|; elsewhere it is close to it.
    Same arguments as ``attention_bwd_fp64``; returns (E_dq, E_dk, E_dv,
    E_delta).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, H, N, d = q.shape
    sigma = abs(_sigma(scale))
    if row_block is None:
        row_block = max(1, (1 << 21) // max(N, 1))
    e_dq = np.empty((B, H, N, d), dtype=np.float64)
    e_dk = np.empty((B, H, N, d), dtype=np.float64)
    e_dv = np.empty((B, H, N, d), dtype=np.float64)
    e_dl = np.empty((B, H, N), dtype=np.float64)

    def one_head(bh):
        b, h = divmod(bh, H)
        qh = q[b, h].astype(np.float64)
        kh = k[b, h].astype(np.float64)
        vh = v[b, h].astype(np.float64)
        doh = do[b, h].astype(np.float64)
        ak = np.abs(kh)
        acc_k = np.zeros((N, d))
        acc_v = np.zeros((N, d))
        for r0 in range(0, N, row_block):
            ids = np.arange(r0, min(r0 + row_block, N))
            s = _masked_scores(qh[ids], ids, kh, _sigma(scale), causal)
            _, e, l = _stable_softmax_parts(s)
            p = e / l[:, None]
            vis = np.isfinite(s) * _SUBNORMAL
            dp = doh[ids] @ vh.T
            dl = (p * dp).sum(axis=1)
            ads = np.abs(p * (dp - dl[:, None])) + vis
            dabs = (np.abs(doh[ids]) * np.abs(p @ vh)).sum(axis=1)
            aq = np.abs(qh[ids])
            e_dq[b, h, ids] = sigma * (ads @ ak + dabs[:, None] * (p @ ak))
            acc_k += sigma * (ads.T @ aq + (p * dabs[:, None]).T @ aq)
            acc_v += (p + vis).T @ np.abs(doh[ids])
            e_dl[b, h, ids] = dabs
        e_dk[b, h] = acc_k
        e_dv[b, h] = acc_v

    nthreads = threads or oracle_threads()
    if nthreads > 1 and B * H > 1:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=nthreads) as ex:
                list(ex.map(one_head, range(B * H)))
    else:
        for bh in range(B * H):
            one_head(bh)
    return e_dq, e_dk, e_dv, e_dl


def attention_bwd_error_std(q, k, v, do, scale, causal=False, threads=None, row_block=None):
    """Per-element statistical error scales S of dQ, dK, dV and delta, float64.

    Not part of what the kernels compute: the scale of a tolerance on their
    result, the root-sum-square form of the bound in
    ``attention_bwd_error_scale``.  Model: each value rounded to fp16 (round
    to nearest) picks up an independent relative error e with
    E[e^2] <= u^2 / 3 (u = 2^-11; e is uniform within half a unit in the
    last place, at most u relative), and a subnormal an absolute error of
    variance (2^-25)^2 / 3.  An error e_j in one factor of a term
    a_j b_j of a sum moves the sum by e_j a_j b_j, so the variance of the
    sum's error is at most (u^2 / 3) sum_j (a_j b_j)^2 -- the same products
    as in the worst-case bound, added in quadrature.  The rounded values
    are those the computation keeps in fp16 on its way:

    * the forward's weights (each P_ij rounded once, shared by the d
      columns of O_i) and its fp16 output O; delta_i = dO_i . O_i taken
      from that O then has error variance <= (u^2/3) D_i with
          D_i = sum_j (P_ij dP_ij)^2 + sum_c (dO_ic O_ic)^2
                + t^2 sum_j M_ij dP_ij^2,                   t = 2^-14;
    * P (for dV) and dS (for dQ, dK), each rounded once; dS also carries
      delta's error, -P_ij err(delta_i), and the fp32 rounding of
      dP_ij - delta_i (2^-24 relative to |dP_ij| and |delta_i|, which only
      matters where they cancel);
    * each gradient's own rounding to fp16.

    Squared scales (error variance <= (u^2 / 3) S^2):
        S_dV^2    = (P^2)^T dO^2 + t^2 M^T dO^2 + dV^2
        S_dQ^2    = sigma^2 [ (dS^2 + t^2 M + F) K^2 + (P K)^2 D ] + dQ^2
        S_dK^2    = sigma^2 [ (dS^2 + t^2 M + F)^T Q^2 + (P^2 D)^T Q^2 ] + dK^2
        S_delta^2 = D
    with squares taken element-wise, M the visibility mask, D broadcast
    over a row's keys and F_ij = 2^-26 d P_ij^2 ((dO^2)(V^2)^T + sum_c
    dO_ic^2 O_ic^2)_ij the fp32 term.  Independent errors then give
    rms(error) <= (u / sqrt 3) rms(S) over many elements; the fp16 rounding
    of values with uniformly distributed mantissas reaches about 0.73 of
    it (E[e^2] ~ 0.18 u^2).  Same arguments as ``attention_bwd_fp64``;
    returns (S_dq, S_dk, S_dv, S_delta).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, H, N, d = q.shape
    sig = _sigma(scale)
    t2 = _SUBNORMAL ** 2
    f32 = _FP32_IN_U16 ** 2 * d
    if row_block is None:
        row_block = max(1, (1 << 21) // max(N, 1))
    s_dq = np.empty((B, H, N, d), dtype=np.float64)
    s_dk = np.empty((B, H, N, d), dtype=np.float64)
    s_dv = np.empty((B, H, N, d), dtype=np.float64)
    s_dl = np.empty((B, H, N), dtype=np.float64)

    def one_head(bh):
        b, h = divmod(bh, H)
        qh = q[b, h].astype(np.float64)
        kh = k[b, h].astype(np.float64)
        vh = v[b, h].astype(np.float64)
        doh = do[b, h].astype(np.float64)
        k2, v2 = kh * kh, vh * vh
        acc_k = np.zeros((N, d))
        acc_v = np.zeros((N, d))
        dk = np.zeros((N, d))
        dv = np.zeros((N, d))
        for r0 in range(0, N, row_block):
            ids = np.arange(r0, min(r0 + row_block, N))
            sc = _masked_scores(qh[ids], ids, kh, sig, causal)
            _, e, l = _stable_softmax_parts(sc)
            p = e / l[:, None]
            vis = np.isfinite(sc).astype(np.float64)
            dor = doh[ids]
            do2 = dor * dor
            dp = dor @ vh.T
            dl = (p * dp).sum(axis=1)
            ds = p * (dp - dl[:, None])
            o = p @ vh
            od2 = (do2 * o * o).sum(axis=1)
            var_dl = (p * p * dp * dp).sum(axis=1) + od2 + t2 * (vis * dp * dp).sum(axis=1)
            q2 = qh[ids] ** 2
            w = ds * ds + t2 * vis + f32 * p * p * (do2 @ v2.T + od2[:, None])
            dq = sig * (ds @ kh)
            s_dq[b, h, ids] = sig * sig * (w @ k2 + (p @ kh) ** 2 * var_dl[:, None]) + dq * dq
            acc_k += sig * sig * (w.T @ q2 + (p * p * var_dl[:, None]).T @ q2)
            acc_v += (p * p + t2 * vis).T @ do2
            dk += sig * (ds.T @ qh[ids])
            dv += p.T @ dor
            s_dl[b, h, ids] = var_dl
        s_dk[b, h] = acc_k + dk * dk
        s_dv[b, h] = acc_v + dv * dv

    nthreads = threads or oracle_threads()
    if nthreads > 1 and B * H > 1:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=nthreads) as ex:
                list(ex.map(one_head, range(B * H)))
    else:
        for bh in range(B * H):
            one_head(bh)
    return np.sqrt(s_dq), np.sqrt(s_dk), np.sqrt(s_dv), np.sqrt(s_dl)
