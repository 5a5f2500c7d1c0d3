// Host-side planning shared by the entry points: workspace sizes and the
// key-range split of the split key/value forward.  Plain C++ (no device
// code), so the argument-checking layer builds and runs without a GPU
// toolchain too.
#include <algorithm>
#include <cstddef>

#include "fa2_launch.h"

namespace fa2 {

namespace {
constexpr int kTileKeys = 64;     // keys per tile of the split key/value kernel
constexpr int kTileQueries = 32;  // queries per workgroup of that kernel
}  // namespace

size_t fa1_workspace_floats(int BH, int N, int d) { return size_t(BH) * N * (size_t(d) + 2); }

SplitPlan plan_splits(int BH, int Nq, int Nk, int requested) {
    const int n_tk = (Nk + kTileKeys - 1) / kTileKeys;
    const int n_qt = (Nq + kTileQueries - 1) / kTileQueries;
    int n = requested;
    if (n <= 0) {
        // One workgroup per CU (256): measured best for d = 64 and 128 at
        // 32..256 heads and 8K..128K keys -- every workgroup does the same
        // work, so a second round only adds a tail.  Every split keeps at
        // least one 64-key tile per wave (four).
        const long target = 256;
        const long groups = long(BH) * n_qt;
        n = int(std::min<long>((target + groups - 1) / groups, std::max(1, n_tk / 4)));
    }
    n = std::max(1, std::min(n, n_tk));
    const int tps = (n_tk + n - 1) / n;
    SplitPlan p;
    p.tiles_per_split = tps;
    p.n_splits = (n_tk + tps - 1) / tps;   // no empty split
    return p;
}

}  // namespace fa2
