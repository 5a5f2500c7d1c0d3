// Test-only stand-ins for the gfx950 launchers, so the C-ABI layer
// (fa2_api.cpp, fa2_plan.cpp) can be built host-only with AddressSanitizer
// and UndefinedBehaviorSanitizer and driven through its argument checks on
// a machine without a GPU.  Any call that gets past the checks reaches one
// of these and gets hipErrorNoDevice back; no device memory is touched.
#include "fa2_launch.h"

namespace fa2 {

hipError_t launch_fwd(const void*, const void*, const void*, void*, float*, int, int, int, float,
                      bool, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_bwd(const void*, const void*, const void*, const void*, const float*,
                      const void*, void*, void*, void*, float*, int, int, int, float, bool,
                      hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_fa1(const void*, const void*, const void*, void*, float*, void*, int, int, int,
                      float, bool, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_splitkv(const void*, const void*, const void*, void*, float*, void*, int, int,
                          int, int, float, const SplitPlan&, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_lse_merge(const float*, const float*, void*, float*, int, int, int, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t noalloc_scratch(hipStream_t, void**) { return hipErrorNoDevice; }

}  // namespace fa2
