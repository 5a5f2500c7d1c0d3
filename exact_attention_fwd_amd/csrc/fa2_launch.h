// Internal interface between the C-ABI entry point (argument checks) and the
// gfx950 kernels.  Not installed; the public interface is include/fa2.h.
#pragma once
#include <hip/hip_runtime.h>

namespace fa2 {

// Launch the forward kernel for already-validated arguments.  Returns the
// HIP error of the launch (hipSuccess on success).
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o,
                      float* lse, int BH, int N, int d, float scale,
                      bool causal, hipStream_t stream);

// Launch the two backward kernels (dQ + delta, then dK/dV) for
// already-validated arguments, in order on `stream`.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      float* delta, int BH, int N, int d, float scale, bool causal,
                      hipStream_t stream);

// The FlashAttention-1 loop order (the comparator): workspace of
// fa1_workspace_floats(BH, N, d) floats (fp32 O, then m, then l).
size_t fa1_workspace_floats(int BH, int N, int d);
hipError_t launch_fa1(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                      int BH, int N, int d, float scale, bool causal, hipStream_t stream);

// Split key/value attention of Nq queries over Nk keys (non-causal): the
// keys split into n_splits ranges of tiles_per_split 64-key tiles.
struct SplitPlan {
    int n_splits = 1;
    int tiles_per_split = 1;
};
// requested <= 0 picks a split count for the shape; the plan never has an
// empty range.
SplitPlan plan_splits(int BH, int Nq, int Nk, int requested);
// ws: plan.n_splits * BH * Nq * (d + 1) floats when plan.n_splits > 1, else unused.
hipError_t launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* ws, int BH, int Nq, int Nk, int d, float scale,
                          const SplitPlan& plan, hipStream_t stream);
// Merge of n_parts partial results [n_parts, rows, d] fp32 with their LSE.
hipError_t launch_lse_merge(const float* opart, const float* lpart, void* o, float* lse,
                            int n_parts, int rows, int d, hipStream_t stream);

}  // namespace fa2
