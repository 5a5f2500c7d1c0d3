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
from the arithmetic: the forward-error bound of a dot product whose factors
were rounded to fp16, |fl(sum a b) - sum a b| <~ u sum |a| |b| with
u = 2^-11.  ``oracle.attention_bwd_error_scale`` gives that scale E per
element (P and dS rounded to fp16, delta taken from the fp16 O, fp16
subnormals); with the fp16 rounding of the result itself the bound reads
u (|G| + E + 2^-14).  Per tensor G:
  max  |G_gpu - G_ref| / (u (|G_ref| + E + 2^-14))  <= 2
  rms  (G_gpu - G_ref) / rms(u (|G_ref| + E + 2^-14)) <= 0.5
An exact emulation of the kernels' roundings stays within 0.9 and 0.23 of
these on random, stress, causal and scale cases (tests/test_bwd_tolerance.py,
which also shows that a dropped or misplaced term exceeds them by far).
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
RMS_RATIO_GRAD = 0.5


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
    rms_ratio: float   # rms(dG) / rms(u (|G| + E + 2^-14))
    rms_rel: float     # rms(dG) / rms(G), for information

    def ok(self) -> bool:
        return self.max_ratio <= MAX_RATIO_GRAD and self.rms_ratio <= RMS_RATIO_GRAD

    def __str__(self):
        return (f"max ratio={self.max_ratio:.3f} rms ratio={self.rms_ratio:.3f} "
                f"(rms rel={self.rms_rel:.2e})")


def grad_diff(g_gpu, g_ref, e_scale) -> GradDiff:
    """Gradient error in units of its rounding-error bound (see above)."""
    err = np.abs(np.asarray(g_gpu, dtype=np.float64) - g_ref)
    den = U16 * (np.abs(g_ref) + e_scale + SUB16)
    if err.size == 0:
        return GradDiff(0.0, 0.0, 0.0)
    rms_ref = float(np.sqrt(np.mean(np.square(g_ref))))
    rms_err = float(np.sqrt(np.mean(np.square(err))))
    return GradDiff(float((err / den).max()), rms_err / float(np.sqrt(np.mean(np.square(den)))),
                    rms_err / rms_ref if rms_ref > 0 else rms_err)


def run_gpu_bwd(q, k, v, do, scale, causal):
    """Forward then backward on the GPU; inputs fp16 numpy arrays.  Returns
    (dq, dk, dv fp16, delta fp32) numpy arrays."""
    import torch
    import exact_attention_fwd_amd as fa2

    tq, tk, tv, tdo = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v, do))
    o, l = fa2.fwd(tq, tk, tv, scale=scale, causal=causal)
    dq, dk, dv, delta = fa2.bwd(tq, tk, tv, o, l, tdo, scale=scale, causal=causal)
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
