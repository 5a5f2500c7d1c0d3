"""Shared helpers for the GPU parity tests: run the HIP path, compare with the
oracle at the tolerances of the attention forward contract.

Gates (fp16 O, fp32 LSE against the float64 oracle):
  max |O_gpu - O_ref|            <= 4e-3
  mean |O_gpu - O_ref|           <= 5e-4
  max |LSE_gpu - LSE_ref| / max(|LSE_ref|, 1) <= 1e-4
The floor of 1 in the LSE denominator keeps rows whose log-sum-exp is near
zero (causal row 0, where LSE is a single scaled score) from turning an
absolute error of ~1e-6 into a spurious relative failure.

Gates of the backward pass (fp16 dQ, dK, dV and fp32 delta against the
float64 gradient oracle).  No tolerance for gradients is given, so it comes
from the arithmetic, the rounding of each value the computation keeps in
fp16 (u = 2^-11), in two forms:
  max  |G_gpu - G_ref| / (u (|G_ref| + E + 2^-14))      <= 2
       E from ``oracle.attention_bwd_error_scale``: the worst-case bound
       u sum |a| |b| of a dot product whose factors were rounded;
  rms  (G_gpu - G_ref) / rms((u / sqrt 3) S)           <= 1
       S from ``oracle.attention_bwd_error_std``: the same products added
       in quadrature, the standard deviation of the error when each
       rounding is an independent relative error of variance <= u^2 / 3.
The rms gate is what rejects arithmetic carried out at lower precision or
biased: an exact emulation of the kernels' fp16 roundings reads 0.6-0.86
of it, P and dS rounded to bf16 2.7-4.5, round-toward-zero conversions
1.7-2.2, a uniform 2^-10 scale error 2.3-2.8 (tests/test_bwd_tolerance.py).
When the backward is handed an O, delta must also meet its definition
delta_i = sum_c dO_ic O_ic for that O within the fp32 bound of a d-term sum
of exact products:
  max |delta_gpu - sum_c dO_ic O_ic| / (d 2^-24 sum_c |dO_ic O_ic|) <= 1.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

MAX_ABS_O = 4e-3
MEAN_ABS_O = 5e-4
MAX_REL_LSE = 1e-4
U16 = 2.0 ** -11          # unit roundoff of fp16
SUB16 = 2.0 ** -14        # fp16 subnormal rounding (2^-25) in units of U16
MAX_RATIO_GRAD = 2.0
RMS_STAT_GRAD = 1.0
U32 = 2.0 ** -24          # unit roundoff of fp32


@dataclass
class Diff:
    max_abs: float
    mean_abs: float
    max_rel_lse: float
    max_rel_lse_unfloored: float

    def ok(self) -> bool:
        return (self.max_abs <= MAX_ABS_O and self.mean_abs <= MEAN_ABS_O
                and self.max_rel_lse <= MAX_REL_LSE)

    def __str__(self):
        return (f"max|dO|={self.max_abs:.3e} mean|dO|={self.mean_abs:.3e} "
                f"max rel dLSE={self.max_rel_lse:.3e} (unfloored {self.max_rel_lse_unfloored:.3e})")


def diff(o_gpu, lse_gpu, o_ref, lse_ref) -> Diff:
    d = np.abs(np.asarray(o_gpu, dtype=np.float64) - o_ref)
    dl = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
    return Diff(float(d.max()), float(d.mean()),
                float((dl / np.maximum(np.abs(lse_ref), 1.0)).max()),
                float((dl / np.maximum(np.abs(lse_ref), 1e-30)).max()))


@dataclass
class GradDiff:
    max_ratio: float   # max |dG| / (u (|G| + E + 2^-14))
    rms_stat: float    # rms(dG) / rms((u / sqrt 3) S)
    rms_rel: float     # rms(dG) / rms(G), for information

    def ok(self) -> bool:
        return self.max_ratio <= MAX_RATIO_GRAD and self.rms_stat <= RMS_STAT_GRAD

    def __str__(self):
        return (f"max ratio={self.max_ratio:.3f} rms stat={self.rms_stat:.3f} "
                f"(rms rel={self.rms_rel:.2e})")


def grad_diff(g_gpu, g_ref, e_scale, s_std) -> GradDiff:
    """Gradient error in units of its rounding-error bounds (see above)."""
    err = np.asarray(g_gpu, dtype=np.float64) - g_ref
    if err.size == 0:
        return GradDiff(0.0, 0.0, 0.0)
    den = U16 * (np.abs(g_ref) + e_scale + SUB16)
    rms_err = float(np.sqrt(np.mean(np.square(err))))
    rms_std = float(np.sqrt(np.mean(np.square(s_std)))) * U16 / np.sqrt(3.0)
    rms_stat = rms_err / rms_std if rms_std > 0 else (0.0 if rms_err == 0 else np.inf)
    rms_ref = float(np.sqrt(np.mean(np.square(g_ref))))
    return GradDiff(float((np.abs(err) / den).max()), rms_stat,
                    rms_err / rms_ref if rms_ref > 0 else rms_err)


def delta_contract(delta_gpu, do, o) -> float:
    """max |delta - sum_c dO_c O_c| over rows, in units of the fp32 bound of
    that d-term sum of exact fp16 products (d 2^-24 sum_c |dO_c O_c|), for
    the O the backward was handed.  <= 1 passes."""
    prod = np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)
    ref = prod.sum(axis=-1)
    bound = prod.shape[-1] * U32 * np.abs(prod).sum(axis=-1)
    err = np.abs(np.asarray(delta_gpu, dtype=np.float64) - ref)
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(ratio.max()) if ratio.size else 0.0


def run_gpu_bwd(q, k, v, do, scale, causal, o=None, lse=None):
    """Backward on the GPU; inputs fp16 numpy arrays.  O and LSE come from the
    GPU forward, unless given (fp16 / fp32 numpy arrays, e.g. the oracle's
    rounded).  Returns (dq, dk, dv fp16, delta fp32) numpy arrays."""
    import torch
    import exact_attention_fwd_amd as fa2

    tq, tk, tv, tdo = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v, do))
    if o is None:
        to, tl = fa2.fwd(tq, tk, tv, scale=scale, causal=causal)
    else:
        to = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float16)).cuda()
        tl = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).cuda()
    dq, dk, dv, delta = fa2.bwd(tq, tk, tv, to, tl, tdo, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy(), delta.cpu().numpy()


def run_gpu(q, k, v, scale, causal, out=None, lse=None):
    """Inputs as fp16 numpy arrays; returns (O fp16, LSE fp32) numpy arrays."""
    import torch
    import exact_attention_fwd_amd as fa2

    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v))
    o, l = fa2.fwd(tq, tk, tv, scale=scale, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.cpu().numpy(), l.cpu().numpy()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()
