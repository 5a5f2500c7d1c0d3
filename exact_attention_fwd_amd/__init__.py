"""FlashAttention-2 forward pass (and its backward) for AMD MI355X (gfx950).

``fwd(q, k, v, scale=None, causal=False) -> (o, lse)`` runs the library's
hand-written gfx950 kernels on torch fp16 tensors, ``bwd(q, k, v, o, lse,
dout, ...) -> (dq, dk, dv, delta)`` their gradients; ``fa2_fwd`` and
``fa2_bwd`` are the C entry points themselves (raw device addresses).
``fwd_fa1`` / ``fa1_fwd`` compute the same forward in the FlashAttention-1
loop order, the comparator of the FA2 kernel.  ``fwd_splitkv`` attends a
short query block to a long key/value set with the keys split across
workgroups (``fwd_splitkv_noalloc``: the same through an entry point that
allocates nothing), and ``lse_merge`` merges partial results over key parts.  The seeded synthetic workloads live in
``exact_attention_fwd_amd.workloads``.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    FA2_ERR_INVALID_ARG,
    FA2_ERR_LAUNCH,
    FA2_ERR_MISALIGNED,
    FA2_ERR_NO_DEVICE,
    FA2_ERR_SCRATCH_LIMIT,
    FA2_NOALLOC_SCRATCH_BYTES,
    FA2_ERR_UNSUPPORTED,
    FA2_OK,
    LIB_PATH,
    Fa2Error,
    bwd,
    fa1_fwd,
    fa1_workspace_bytes,
    fa2_bwd,
    fa2_fwd,
    fa2_fwd_splitkv,
    fa2_fwd_splitkv_noalloc,
    fa2_lse_merge,
    fa2_splitkv_splits,
    fa2_splitkv_workspace_bytes,
    fa2_last_hip_error,
    fa2_status_string,
    fa2_version,
    fwd,
    fwd_fa1,
    fwd_splitkv,
    fwd_splitkv_noalloc,
    load_library,
    lse_merge,
)
