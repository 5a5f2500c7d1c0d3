"""Plain float64 CPU attention: the oracle the HIP kernels are checked against.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code may
import or call anything here.

Sources (cited by page title and section; the pages are web articles):

* "3.6 Attention I -- the memory problem and FlashAttention principles"
  (a textbook chapter; cited below as [Attn-I]):
  - 3.6.2: scaled dot-product attention of one head, two GEMMs with a
    row-wise softmax between them;
  - 3.6.4: the stable softmax (subtract the row max) and the online-softmax
    recurrence over key blocks (running max m, running sum l, running output
    O, correction factor alpha = exp(m_old - m_new), one division at the end);
  - 3.6.5: the hand-worked example used as a pin;
  - 3.6.6: the tile loop and the causal rule (key blocks in the future are
    skipped, the diagonal block is partly masked);
  - 3.6.7: the row statistic kept for the backward pass, L = m + log l;
  - 3.6.10: the two pitfalls used as negative controls (rescaling only one of
    l and O; dropping the max shift).
* "FlashAttention-2 from scratch in CuTe" (a jeff.news summary; [CuTe-FA2]),
  section on the kernel structure: P = Q K^T / sqrt(d_h), softmax, O = S V,
  fp16 inputs with fp32 accumulation.
* "A learning journey: CUDA, Triton, Flash Attention" (GPU MODE lecture 50
  notes; [GPU-MODE-50]): the one-query-block FA2 pseudocode, which returns
  O / l together with m and l.

Readings taken where the pages are silent:

* the scale used is the float32 value that crosses the C ABI, widened to
  float64 exactly (``sigma = float(np.float32(scale))``);
* causal means key j is visible to query i iff j <= i (equal query and key
  lengths, top-left aligned);
* LSE is the natural log-sum-exp of the *scaled* scores over visible keys,
  LSE = m + ln(l);
* O is returned in float64, not rounded to fp16;
* a block in which every score of a row is masked contributes nothing (the
  online variant uses shift 0 when the running max is still -inf, so that
  -inf - (-inf) never occurs).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "attention_fp64",
    "attention_probs_fp64",
    "online_softmax_attention",
    "brute_force_attention",
    "oracle_threads",
]


def oracle_threads() -> int:
    """Host threads the oracle uses: every core this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover - non-Linux
        return max(1, os.cpu_count() or 1)


def _sigma(scale: float) -> float:
    """The scale as the kernel receives it: an fp32 value, widened exactly."""
    return float(np.float32(scale))


def _masked_scores(q_rows: np.ndarray, row_ids: np.ndarray, k: np.ndarray,
                   sigma: float, causal: bool) -> np.ndarray:
    """S = sigma * Q_rows K^T with future keys set to -inf.

    [Attn-I] 3.6.2 (the first GEMM, scaled) and 3.6.6 (causal: key j is
    masked for j > i).  Shapes: q_rows [R, d], k [N, d] -> [R, N], float64.
    """
    s = sigma * (q_rows @ k.T)
    if causal:
        keys = np.arange(k.shape[0])
        s[keys[None, :] > row_ids[:, None]] = -np.inf
    return s


def _stable_softmax_parts(s: np.ndarray):
    """Row max m, unnormalised weights exp(S - m) and their sum l.

    [Attn-I] 3.6.4, the stable softmax: m = max_j x_j, weights exp(x_j - m),
    denominator sum_k exp(x_k - m).  Every row has at least one finite score
    (causal row i always sees key i), so m is finite.
    """
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    return m, p, l


def _attention_rows(q_rows, row_ids, k, v, sigma, causal):
    """O, LSE, m, l for a block of query rows of one (batch, head).

    O = (sum_j exp(s_ij - m_i) v_j) / l_i        [Attn-I] 3.6.2 + 3.6.4
    LSE = m + ln l                                 [Attn-I] 3.6.7
    """
    s = _masked_scores(q_rows, row_ids, k, sigma, causal)
    m, p, l = _stable_softmax_parts(s)
    o = (p @ v) / l[:, None]
    lse = m + np.log(l)
    return o, lse, m, l


def attention_fp64(q, k, v, scale, causal=False, rows=None, return_stats=False,
                   threads=None, row_block=None):
    """Materialised softmax attention in float64, the definition itself.

    Arguments
      q, k, v : arrays [B, H, N, d] (fp16 inputs are widened exactly).  Without
                the causal mask the keys may be a different number Nk: q is
                [B, H, N, d], k and v [B, H, Nk, d] (a short query block
                against a long key/value cache; every query sees every key).
      scale   : the softmax scale (1/sqrt(d) in the workloads); used as the
                fp32 value the kernel receives.
      causal  : mask key j for query i when j > i.
      rows    : None for every query row, or an integer array [R] (the same
                rows for every head) or [B, H, R] (rows per head).
      return_stats : also return the row max m and row sum l.
      threads : worker threads over (b, h); BLAS is held to one thread each.
      row_block : query rows per materialised score block (memory bound).

    Returns O [B, H, R, d] float64 and LSE [B, H, R] float64 (R = N when rows
    is None), plus m and l [B, H, R] when return_stats is set.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if causal and q.shape[2] != k.shape[2]:
        raise ValueError("causal attention needs as many queries as keys")
    B, H, N, d = q.shape
    sigma = _sigma(scale)
    if rows is None:
        row_idx = np.broadcast_to(np.arange(N), (B, H, N))
    else:
        r = np.asarray(rows, dtype=np.int64)
        row_idx = np.broadcast_to(r, (B, H, r.shape[-1])) if r.ndim == 1 else r
        if row_idx.shape[:2] != (B, H):
            raise ValueError("rows must be [R] or [B, H, R]")
        if row_idx.size and (row_idx.min() < 0 or row_idx.max() >= N):
            raise ValueError("row index out of range")
    R = row_idx.shape[-1]
    if row_block is None:
        row_block = max(1, (1 << 23) // max(N, 1))  # ~64 MiB of fp64 scores
    o_out = np.empty((B, H, R, d), dtype=np.float64)
    lse_out = np.empty((B, H, R), dtype=np.float64)
    m_out = np.empty((B, H, R), dtype=np.float64)
    l_out = np.empty((B, H, R), dtype=np.float64)

    def one_head(bh):
        b, h = divmod(bh, H)
        qh = q[b, h].astype(np.float64)
        kh = k[b, h].astype(np.float64)
        vh = v[b, h].astype(np.float64)
        ids = row_idx[b, h]
        for r0 in range(0, R, row_block):
            sel = ids[r0:r0 + row_block]
            o, lse, m, l = _attention_rows(qh[sel], sel, kh, vh, sigma, causal)
            o_out[b, h, r0:r0 + row_block] = o
            lse_out[b, h, r0:r0 + row_block] = lse
            m_out[b, h, r0:r0 + row_block] = m
            l_out[b, h, r0:r0 + row_block] = l

    nthreads = threads or oracle_threads()
    if nthreads > 1 and B * H > 1:
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(limits=1)
        except ImportError:  # pragma: no cover - threadpoolctl is installed
            limiter = None
        try:
            with ThreadPoolExecutor(max_workers=nthreads) as ex:
                list(ex.map(one_head, range(B * H)))
        finally:
            if limiter is not None:
                limiter.restore_original_limits()
    else:
        for bh in range(B * H):
            one_head(bh)
    if return_stats:
        return o_out, lse_out, m_out, l_out
    return o_out, lse_out


def attention_probs_fp64(q, k, scale, causal=False):
    """The materialised, normalised softmax matrix [B, H, N, N] (tiny shapes).

    Built from the same steps as ``attention_fp64`` so that its invariants
    (rows sum to one, masked entries are zero) check the oracle's own
    arithmetic.  [Attn-I] 3.6.2, 3.6.4.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    B, H, N, _ = q.shape
    sigma = _sigma(scale)
    out = np.empty((B, H, N, N), dtype=np.float64)
    ids = np.arange(N)
    for b in range(B):
        for h in range(H):
            s = _masked_scores(q[b, h].astype(np.float64), ids,
                               k[b, h].astype(np.float64), sigma, causal)
            _, p, l = _stable_softmax_parts(s)
            out[b, h] = p / l[:, None]
    return out


def online_softmax_attention(q, k, v, scale, causal=False, row_ids=None,
                             block_size=None, blocks=None, order=None,
                             rescale="both", max_shift=True, trace=False):
    """The online-softmax recurrence over key blocks, float64, one head.

    Used only to check the oracle (its result must not depend on block size
    or order).  It follows [Attn-I] 3.6.4 / 3.6.6 and the [GPU-MODE-50]
    pseudocode: state (m, l, O) starts at (-inf, 0, 0); for each key block
      m_tilde = rowmax(S_blk),  m_new = max(m, m_tilde),
      alpha = exp(m - m_new),   p = exp(S_blk - m_new),
      l = alpha * l + rowsum(p),  O = alpha * O + p V_blk,  m = m_new;
    finally O / l and LSE = m + ln l ([Attn-I] 3.6.7).

    Arguments
      q [M, d] query rows with absolute indices ``row_ids`` (default 0..M-1),
      k, v [N, d]; ``blocks`` is a list of key-index arrays, or ``block_size``
      splits 0..N-1 into consecutive blocks; ``order`` permutes the blocks.
      Negative controls ([Attn-I] 3.6.10): ``rescale`` = "l_only" or
      "o_only" applies alpha to one of l, O only; ``max_shift=False`` drops
      the max subtraction (exp of the raw scores).
      ``trace`` returns the per-block states as well.

    Returns (O [M, d], LSE [M]) or (O, LSE, states).
    """
    if rescale not in ("both", "l_only", "o_only"):
        raise ValueError("rescale must be 'both', 'l_only' or 'o_only'")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, N = q.shape[0], k.shape[0]
    sigma = _sigma(scale)
    row_ids = np.arange(M) if row_ids is None else np.asarray(row_ids)
    if blocks is None:
        bs = N if block_size is None else int(block_size)
        blocks = [np.arange(j, min(j + bs, N)) for j in range(0, N, bs)]
    else:
        blocks = [np.asarray(b, dtype=np.int64) for b in blocks]
    if order is not None:
        blocks = [blocks[i] for i in order]

    m = np.full(M, -np.inf)
    l = np.zeros(M)
    o = np.zeros((M, v.shape[1]))
    states = []
    with np.errstate(over="ignore", invalid="ignore"):
        for blk in blocks:
            s = sigma * (q @ k[blk].T)
            if causal:
                s[blk[None, :] > row_ids[:, None]] = -np.inf
            m_tilde = s.max(axis=1) if s.shape[1] else np.full(M, -np.inf)
            m_new = np.maximum(m, m_tilde)
            if max_shift:
                # A row with nothing visible yet keeps shift 0: its weights
                # and alpha are exp(-inf) = 0 and the state stays (-inf, 0, 0).
                shift = np.where(np.isneginf(m_new), 0.0, m_new)
            else:
                shift = np.zeros(M)
            alpha = np.exp(np.where(np.isneginf(m), -np.inf, m - shift))
            if not max_shift:
                alpha = np.where(np.isneginf(m), 0.0, 1.0)
            p = np.exp(s - shift[:, None])
            l = (alpha * l if rescale in ("both", "l_only") else l) + p.sum(axis=1)
            o = (alpha[:, None] * o if rescale in ("both", "o_only") else o) + p @ v[blk]
            if trace:
                states.append(dict(m_tilde=m_tilde.copy(), m_new=m_new.copy(),
                                   alpha=alpha.copy(), p=p.copy(), l=l.copy(),
                                   o=o.copy()))
            m = m_new
        out = o / l[:, None]
        lse = (m if max_shift else 0.0) + np.log(l)
    if trace:
        return out, lse, states
    return out, lse


def brute_force_attention(q, k, v, scale, causal=False):
    """Pure-Python attention for tiny inputs: nested loops, math.exp, math.fsum.

    The same definition as ``attention_fp64`` ([Attn-I] 3.6.2, 3.6.4, 3.6.7)
    written with exactly rounded sums and no numpy arithmetic, so that a slip
    in the vectorised oracle (a transposed operand, a wrong mask index, a
    missing term) shows up as a mismatch.  Inputs are nested lists or arrays
    [B, H, N, d] (k, v may have another length when not causal); returns
    (O, LSE) as nested lists of floats.
    """
    sigma = _sigma(scale)
    q = np.asarray(q).astype(np.float64).tolist()
    k = np.asarray(k).astype(np.float64).tolist()
    v = np.asarray(v).astype(np.float64).tolist()
    o_all, lse_all = [], []
    for b in range(len(q)):
        o_b, lse_b = [], []
        for h in range(len(q[b])):
            qs, ks, vs = q[b][h], k[b][h], v[b][h]
            n, nk, d = len(qs), len(ks), len(qs[0])
            o_h, lse_h = [], []
            for i in range(n):
                visible = [j for j in range(nk) if not (causal and j > i)]
                s = {j: sigma * math.fsum(qs[i][t] * ks[j][t] for t in range(d))
                     for j in visible}
                m = max(s.values())
                w = {j: math.exp(s[j] - m) for j in visible}
                l = math.fsum(w.values())
                o_h.append([math.fsum(w[j] * vs[j][t] for j in visible) / l
                            for t in range(d)])
                lse_h.append(m + math.log(l))
            o_b.append(o_h)
            lse_b.append(lse_h)
        o_all.append(o_b)
        lse_all.append(lse_b)
    return o_all, lse_all
