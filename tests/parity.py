"""Shared helpers for the GPU parity tests: run the HIP path, compare with the
oracle at the tolerances of the attention forward contract.

Gates (fp16 O, fp32 LSE against the float64 oracle):
  max |O_gpu - O_ref|            <= 4e-3
  mean |O_gpu - O_ref|           <= 5e-4
  max |LSE_gpu - LSE_ref| / max(|LSE_ref|, 1) <= 1e-4
The floor of 1 in the LSE denominator keeps rows whose log-sum-exp is near
zero (causal row 0, where LSE is a single scaled score) from turning an
absolute error of ~1e-6 into a spurious relative failure.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

MAX_ABS_O = 4e-3
MEAN_ABS_O = 5e-4
MAX_REL_LSE = 1e-4


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
