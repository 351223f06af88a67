// Host-only stand-ins for the kernel launchers, so that the host control
// plane (host.cpp) can be built with g++ and the address / undefined-
// behaviour sanitizers and exercised on a machine without a GPU.  Every
// launcher reports success without touching memory.
#include "../../non_uniform_paged_amd/csrc/kernels.h"

namespace nup {
bool supported_shape(int, int) { return true; }
int partial_blocks_per_cu(int, int, int) { return 2; }
hipError_t launch_partial(const PartialArgs &, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_merge(const MergeArgs &, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_append(const AppendArgs &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_score(const ScoreArgs &, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_select(const SelectArgs &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_centroid_select(const CentroidArgs &, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_gather_index(const GatherIndexArgs &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_gather_runs(const GatherRunsArgs &, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_fill(int32_t *, int, int32_t, hipStream_t) { return hipSuccess; }
hipError_t launch_apply_patches(int32_t *, const int32_t *, const int32_t *, int, int, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_probe_copy(const void *, void *, size_t, hipStream_t) { return hipSuccess; }
hipError_t scratch_buffer(int, void **ptr) {
    *ptr = nullptr;
    return hipErrorNoDevice;
}
hipError_t launch_probe_read(const void *, size_t, uint32_t *, hipStream_t) { return hipSuccess; }
}  // namespace nup
