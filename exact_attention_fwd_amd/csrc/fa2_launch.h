// Internal interface between the C-ABI entry point (argument checks) and the
// gfx950 kernels.  Not installed; the public interface is include/fa2.h.
#pragma once
#include <hip/hip_runtime.h>

namespace fa2 {

// Head group for causal grids (head_tile_of): the largest power of two g
// with g * n_tiles at most the workgroups an XCD (32 of the 256 CUs) runs at
// once, wgs_per_cu each, and with each XCD's range of n_wg / 8 logical ids a
// whole number of groups; 1 when none fits.
inline int causal_group(int n_tiles, int n_wg, int wgs_per_cu) {
    if (n_wg % 8 != 0 || n_tiles <= 0) return 1;
    const long at_once = 32L * wgs_per_cu;
    int g = 1;
    while (2L * g * n_tiles <= at_once) g *= 2;
    while (g > 1 && (n_wg / 8) % (g * n_tiles) != 0) g /= 2;
    return g;
}

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
// The calling device's copy of the library's fixed scratch buffer
// (FA2_NOALLOC_SCRATCH_BYTES; the device of `stream`, or the current one for
// the null stream).  The address is looked up with hipGetSymbolAddress on
// the first call for a device and kept; nothing is allocated.
hipError_t noalloc_scratch(hipStream_t stream, void** out);
// Merge of n_parts partial results [n_parts, rows, d] fp32 with their LSE.
hipError_t launch_lse_merge(const float* opart, const float* lpart, void* o, float* lse,
                            int n_parts, int rows, int d, hipStream_t stream);

}  // namespace fa2
