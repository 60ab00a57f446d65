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
// Debugging aids among them: ZR_FORCE_PATH overrides the kernels' choice of
// access path or tile shape where they have one, and ZR_DEBUG makes every call
// wait for its stream after its launches (outside stream capture), so a fault
// in a kernel is reported by the call that launched it.
enum ForcePath {
    kPathAuto = 0,     // each kernel's own choice
    kPathElement = 1,  // element-wise folds and copies (reduce-scatter, discrete
                       // reduce-scatter, all-reduce, all-gather)
    kPathSmall = 2,    // one-slice tiles for every ring-order reduce-scatter
    kPathLarge = 3,    // full tiles for every reduce-scatter, however small
};
struct Tuning {
    int ar_nontemporal;    // fused all-reduce: streaming (non-temporal) loads and stores
    int ag_nontemporal;    // all-gather
    int max_grid;          // blocks per launch at most (ZR_MAX_GRID, default 2^30): every
                           // kernel launches one block per tile up to it, and its blocks
                           // stride over the tiles beyond it
    int force_path;        // ZR_FORCE_PATH: element | small | large (a ForcePath)
    int rs_pairs;          // ZR_RS_PAIRS: reduce-scatter tiles by pairs of chunks (1) or chunk by chunk (0)
    int debug;             // ZR_DEBUG: 1 = wait for the stream after each call's launches
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

// A reduce-scatter prepared once (launch geometry and kernel chosen) and
// launched many times. rs_plan_build returns NULL when host memory runs out.
struct RsPlan;
RsPlan* rs_plan_build(int K, const ConstPtrs& in, zr_dtype in_dt, int64_t N, const MutPtrs& out,
                      zr_dtype out_dt, int shift, int flags, zr_order order);
hipError_t rs_plan_launch(const RsPlan* plan, hipStream_t stream);
void rs_plan_free(RsPlan* plan);

hipError_t launch_allreduce_fused(int K, const ConstPtrs& in, const MutPtrs& out, zr_dtype dt,
                                  int64_t N, int average, zr_order order, hipStream_t stream);

// segs: up to kAgSegsPerLaunch segments per call.
hipError_t launch_all_gather(int K, const ConstPtrs& shards, const MutPtrs& fulls, zr_dtype dt,
                             const zr_seg* segs, int n_segs, int shift, hipStream_t stream);
// Any number of segments in one launch, their table staged to `ws` (at least
// ag_table_bytes(n_segs) bytes) on `stream` first.
hipError_t launch_all_gather_ws(int K, const ConstPtrs& shards, const MutPtrs& fulls, zr_dtype dt,
                                const zr_seg* segs, int n_segs, int shift, void* ws,
                                hipStream_t stream);

// Device descriptor tables. A call whose fragment (or segment) table does not
// fit one kernel-argument block either goes out as several argument launches
// or, given a workspace, as one launch that reads the whole table from it.
// The host builds the table as a byte image whose internal pointers already
// hold the workspace's device addresses; staging copies the image there.
// Every table is laid out in 8-byte words (sizes below in bytes).
constexpr size_t kWsAlign = 256;

// Discrete reduce-scatter: first tiles int64[nseg + 1], segment records
// int32[3 * nseg] (entry, chunk, head), entry records int64[2 * nent]
// (offset, size), rank pointers [K * nent].
struct RsfLayout {
    size_t tile0, seg, ent, ptr, bytes;
    RsfLayout(int K, int64_t nent, int64_t nseg) {
        tile0 = 0;
        seg = tile0 + 8 * (size_t)(nseg + 1);
        ent = seg + ((12 * (size_t)nseg + 7) & ~(size_t)7);
        ptr = ent + 16 * (size_t)nent;
        bytes = ptr + 8 * (size_t)K * (size_t)nent;
    }
};
// Flatten: first tiles int64[nent + 1], tiles per rank int64[nent], entry
// records int64[2 * nent] (offset, size), source pointers [K * nent].
struct FlatLayout {
    size_t tile0, tpr, ent, src, bytes;
    FlatLayout(int K, int64_t nent) {
        tile0 = 0;
        tpr = tile0 + 8 * (size_t)(nent + 1);
        ent = tpr + 8 * (size_t)nent;
        src = ent + 16 * (size_t)nent;
        bytes = src + 8 * (size_t)K * (size_t)nent;
    }
};
// All-gather: first tiles int64[nseg + 1], then kAgSegBytes per segment record.
constexpr size_t kAgSegBytes = 48;
inline size_t rsf_table_bytes(int K, int64_t n_entries, int64_t n_segs) {
    return RsfLayout(K, n_entries, n_segs).bytes;
}
inline size_t flatten_table_bytes(int K, int64_t n_entries) { return FlatLayout(K, n_entries).bytes; }
inline size_t ag_table_bytes(int64_t n_segs) { return 8 * (size_t)(n_segs + 1) + kAgSegBytes * (size_t)n_segs; }
// Copies a table image to the workspace: asynchronously on `stream`, or with a
// blocking copy when `stream_order` is false (plan creation).
hipError_t stage_table(void* ws, const void* image, size_t bytes, hipStream_t stream, bool stream_order);

// Discrete reduce-scatter over fragment entries (any count): a plan holds the
// launches' argument blocks, built once and launched many times. With `ws`
// non-null and more than one argument launch needed, the plan instead holds
// one launch whose table image (table_bytes, host copy in table_image) is to
// be staged to `ws` before the launch. rsf_plan_build returns NULL when host
// memory runs out.
struct RsfPlan;
RsfPlan* rsf_plan_build(int K, const FragEntry* entries, int n_entries, int64_t N, zr_dtype in_dt,
                        const MutPtrs& out, zr_dtype out_dt, int shift, int flags, zr_order order,
                        void* ws);
size_t rsf_plan_table_bytes(const RsfPlan* plan);   // 0: argument launches only
const void* rsf_plan_table_image(const RsfPlan* plan);
int rsf_plan_launch_count(const RsfPlan* plan);
hipError_t rsf_plan_launch(const RsfPlan* plan, hipStream_t stream);
void rsf_plan_free(RsfPlan* plan);

// Device address, on the current device, of the file-scope staging array of
// ZR_NOALLOC_TABLE_BYTES bytes that zr_reduce_scatter_frags_noalloc stages its
// table in (looked up once per device with hipGetSymbolAddress).
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void** ptr);

// Bucket flatten over fragment entries, planned the same way: argument
// launches of kFlatEntriesPerLaunch (or fewer) entries, an entry of more than
// 2^28 / K tiles of 4 KiB per rank cut into pieces of that many (so tile
// numbers fit 32 bits), or, with `ws`, one launch over a staged table of the
// uncut entries.
struct FlatPlan;
FlatPlan* flat_plan_build(int K, const FragEntry* entries, int n_entries, const MutPtrs& buckets,
                          int elem_bytes, void* ws);
size_t flat_plan_table_bytes(const FlatPlan* plan);
const void* flat_plan_table_image(const FlatPlan* plan);
int flat_plan_launch_count(const FlatPlan* plan);
hipError_t flat_plan_launch(const FlatPlan* plan, hipStream_t stream);
void flat_plan_free(FlatPlan* plan);

}  // namespace zr
