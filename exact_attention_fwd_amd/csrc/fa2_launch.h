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

}  // namespace fa2
