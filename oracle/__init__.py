"""CPU oracle for the FlashAttention-2 forward pass and its gradients.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: it is used by ``tests/``, by the ``cpu_baseline`` leg of
``bench.py`` and by ``__graft_entry__.smoke()`` to check the HIP kernels.  It
shares no code, header, table or helper with ``exact_attention_fwd_amd``; the
two meet only in the seeded input generators, which hold none of the method's
arithmetic.

Everything here is plain float64 numpy (plus one pure-Python brute force for
tiny cases).  See ``oracle.attention`` (forward), ``oracle.attention_bwd``
(gradients) and ``oracle.merge`` (merging partial results over key parts) for
the functions and the passages of the pages each one follows.
"""
from .attention import (
    attention_fp64,
    attention_probs_fp64,
    online_softmax_attention,
    brute_force_attention,
)
from .attention_bwd import attention_bwd_fp64
from .merge import merge_lse_fp64

__all__ = [
    "attention_fp64",
    "attention_probs_fp64",
    "online_softmax_attention",
    "brute_force_attention",
    "attention_bwd_fp64",
    "merge_lse_fp64",
]
