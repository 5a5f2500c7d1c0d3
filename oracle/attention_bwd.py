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

__all__ = ["attention_bwd_fp64", "attention_bwd_error_scale"]

# Absolute rounding error of an fp16 subnormal (2^-25) in units of the
# relative one (u = 2^-11).
_SUBNORMAL = 2.0 ** -14


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
