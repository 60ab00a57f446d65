// Link stubs for a host-only build of the C-ABI layer (zr_abi.cpp,
// zr_sched.cpp, zr_prefetch.cpp, zr_cost.cpp compiled with g++ under the
// address and undefined-behaviour sanitizers). Test infrastructure only: the
// CPU tests that run against that build never reach a kernel launch (every
// call they make fails validation, has no work, or builds a plan it does not
// launch), so the launch functions of the HIP sources are replaced by ones
// that report the operation unsupported.
#include "zr_internal.hpp"

namespace zr {

hipError_t launch_reduce_scatter(int, const ConstPtrs&, zr_dtype, int64_t, const MutPtrs&, zr_dtype, int,
                                 int, zr_order, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_allreduce_fused(int, const ConstPtrs&, const MutPtrs&, zr_dtype, int64_t, int, zr_order,
                                  hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_all_gather(int, const ConstPtrs&, const MutPtrs&, zr_dtype, const zr_seg*, int, int,
                             hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_flatten(int, const FragEntry*, int, const MutPtrs&, int, hipStream_t) {
    return hipErrorNotSupported;
}

struct RsfPlan {
    int n_entries;
};

RsfPlan* rsf_plan_build(int, const FragEntry*, int n_entries, int64_t, zr_dtype, const MutPtrs&, zr_dtype,
                        int, int, zr_order) {
    return new RsfPlan{n_entries};
}

hipError_t rsf_plan_launch(const RsfPlan*, hipStream_t) { return hipErrorNotSupported; }

void rsf_plan_free(RsfPlan* plan) { delete plan; }

}  // namespace zr
