// Internal launch interface between the C-ABI layer (zr_abi.cpp,
// zr_sched.cpp) and the HIP kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zr.h"

namespace zr {

constexpr int kMaxRanks = ZR_MAX_RANKS;
constexpr int kAgSegsPerLaunch = 32;   // segments carried in one all-gather launch
constexpr int kFlatPtrsPerLaunch = 256;    // source pointers of fragments in one flatten launch
constexpr int kFlatEntriesPerLaunch = 32;  // fragments in one flatten launch
constexpr int kRsfPtrsPerLaunch = 256;   // rank pointers of fragments in one discrete-RS launch
constexpr int kRsfEntriesPerLaunch = 32; // fragments in one discrete-RS launch
constexpr int kRsfSegsPerLaunch = 96;    // (fragment, chunk) segments in one discrete-RS launch

// Rank pointer tables travel by value in kernel arguments (K <= 64 -> 512 B).
struct ConstPtrs {
    const void* p[kMaxRanks];
};
struct MutPtrs {
    void* p[kMaxRanks];
};

// One fragment of a flatten or a discrete reduce-scatter: its K rank
// pointers (all null for the zero padding after the last fragment), its
// offset in the (virtual) bucket, and its size.
struct FragEntry {
    const void* ptr[kMaxRanks];
    int64_t off, n;
};

// Knobs read once from the environment (for tuning sweeps and tests);
// defaults are the measured best.
struct Tuning {
    int ar_nontemporal;    // fused all-reduce: streaming (non-temporal) loads and stores
    int ag_nontemporal;    // all-gather
    int max_grid;          // blocks per launch at most (ZR_MAX_GRID, default 2^30): every
                           // kernel launches one block per tile up to it, and its blocks
                           // stride over the tiles beyond it
};
const Tuning& tuning();
// Blocks for a launch of `tiles` tiles: one per tile, at most tuning().max_grid.
inline int grid_for(int64_t tiles, int64_t cap_divisor = 1) {
    const int64_t cap = tuning().max_grid / cap_divisor > 0 ? tuning().max_grid / cap_divisor : 1;
    return (int)(tiles < cap ? tiles : cap);
}
int device_cu_count();  // CUs of the current device (cached per device)

// flags: ZR_AVERAGE | ZR_ACCUMULATE
hipError_t launch_reduce_scatter(int K, const ConstPtrs& in, zr_dtype in_dt, int64_t N,
                                 const MutPtrs& out, zr_dtype out_dt, int shift, int flags,
                                 zr_order order, hipStream_t stream);

hipError_t launch_allreduce_fused(int K, const ConstPtrs& in, const MutPtrs& out, zr_dtype dt,
                                  int64_t N, int average, zr_order order, hipStream_t stream);

// segs: up to kAgSegsPerLaunch segments per call.
hipError_t launch_all_gather(int K, const ConstPtrs& shards, const MutPtrs& fulls, zr_dtype dt,
                             const zr_seg* segs, int n_segs, int shift, hipStream_t stream);

// Discrete reduce-scatter over fragment entries (any count): the launches'
// argument blocks are built once into a plan and can be launched many times.
// rsf_plan_build returns NULL when host memory runs out.
struct RsfPlan;
RsfPlan* rsf_plan_build(int K, const FragEntry* entries, int n_entries, int64_t N, zr_dtype in_dt,
                        const MutPtrs& out, zr_dtype out_dt, int shift, int flags, zr_order order);
hipError_t rsf_plan_launch(const RsfPlan* plan, hipStream_t stream);
void rsf_plan_free(RsfPlan* plan);

// Any number of entries, each with at most 2^28 / K tiles of 4 KiB per
// rank; launched kFlatEntriesPerLaunch (or fewer) at a time.
hipError_t launch_flatten(int K, const FragEntry* entries, int n_entries, const MutPtrs& buckets,
                          int elem_bytes, hipStream_t stream);

}  // namespace zr
