// Link stubs for a host-only build of the C-ABI layer (zr_abi.cpp,
// zr_sched.cpp, zr_prefetch.cpp, zr_cost.cpp compiled with g++ under the
// address and undefined-behaviour sanitizers). Test infrastructure only: the
// CPU tests that run against that build never reach a kernel launch (every
// call they make fails validation, has no work, or builds a plan it does not
// launch), so the launch functions of the HIP sources are replaced by ones
// that report the operation unsupported, and the plan builders by ones that
// only count launches and size the staged table.
#include <vector>

#include "zr_internal.hpp"

namespace zr {

hipError_t launch_reduce_scatter(int, const ConstPtrs&, zr_dtype, int64_t, const MutPtrs&, zr_dtype, int,
                                 int, zr_order, hipStream_t) {
    return hipErrorNotSupported;
}

struct RsPlan {
    int K;
};
RsPlan* rs_plan_build(int K, const ConstPtrs&, zr_dtype, int64_t, const MutPtrs&, zr_dtype, int, int, zr_order) {
    (void)tuning();  // the library's builder reads the environment settings here
    return new RsPlan{K};
}
hipError_t rs_plan_launch(const RsPlan*, hipStream_t) { return hipErrorNotSupported; }
void rs_plan_free(RsPlan* plan) { delete plan; }

hipError_t launch_allreduce_fused(int, const ConstPtrs&, const MutPtrs&, zr_dtype, int64_t, int, zr_order,
                                  hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_all_gather(int, const ConstPtrs&, const MutPtrs&, zr_dtype, const zr_seg*, int, int,
                             hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_all_gather_ws(int, const ConstPtrs&, const MutPtrs&, zr_dtype, const zr_seg*, int, int, void*,
                                hipStream_t) {
    return hipErrorNotSupported;
}

// Plans that launch nothing but make the same host-side decisions as the
// library's: min(32, 256 / K) fragments per argument launch (the padding
// entry riding in a spare slot of the last one), and with a workspace and
// more than one such launch, one launch over a staged table of the real
// layout's size (its pieces counted at their upper bound, entries + K - 1).
namespace {
struct StubPlan {
    int launches = 0;
    std::vector<unsigned char> image;
};
StubPlan* stub_plan(int K, const FragEntry* entries, int n_entries, void* ws, bool rsf) {
    int frags = 0;
    for (int i = 0; i < n_entries; ++i) frags += entries[i].ptr[0] != nullptr;
    const int per = (256 / K) < 32 ? (256 / K) : 32;
    StubPlan* p = new StubPlan();
    p->launches = frags > 0 ? (frags + per - 1) / per : (n_entries > 0 ? 1 : 0);
    if (ws && p->launches > 1) {
        p->launches = 1;
        p->image.assign(rsf ? rsf_table_bytes(K, n_entries, n_entries + K - 1)
                            : flatten_table_bytes(K, n_entries), 0);
    }
    return p;
}
}  // namespace

struct RsfPlan : StubPlan {};

RsfPlan* rsf_plan_build(int K, const FragEntry* entries, int n_entries, int64_t, zr_dtype, const MutPtrs&,
                        zr_dtype, int, int, zr_order, void* ws) {
    StubPlan* s = stub_plan(K, entries, n_entries, ws, true);
    RsfPlan* p = new RsfPlan();
    p->launches = s->launches;
    p->image.swap(s->image);
    delete s;
    return p;
}
size_t rsf_plan_table_bytes(const RsfPlan* p) { return p->image.size(); }
const void* rsf_plan_table_image(const RsfPlan* p) { return p->image.data(); }
int rsf_plan_launch_count(const RsfPlan* p) { return p->launches; }
hipError_t rsf_plan_launch(const RsfPlan*, hipStream_t) { return hipErrorNotSupported; }
void rsf_plan_free(RsfPlan* plan) { delete plan; }

struct FlatPlan : StubPlan {};

FlatPlan* flat_plan_build(int K, const FragEntry* entries, int n_entries, const MutPtrs&, int, void* ws) {
    StubPlan* s = stub_plan(K, entries, n_entries, ws, false);
    FlatPlan* p = new FlatPlan();
    p->launches = s->launches;
    p->image.swap(s->image);
    delete s;
    return p;
}
size_t flat_plan_table_bytes(const FlatPlan* p) { return p->image.size(); }
const void* flat_plan_table_image(const FlatPlan* p) { return p->image.data(); }
int flat_plan_launch_count(const FlatPlan* p) { return p->launches; }
hipError_t flat_plan_launch(const FlatPlan*, hipStream_t) { return hipErrorNotSupported; }
void flat_plan_free(FlatPlan* plan) { delete plan; }

hipError_t noalloc_scratch(void**) { return hipErrorNotSupported; }

}  // namespace zr
