// Host planning of the discrete reduce-scatter: segments, heads, argument
// launches and staged tables, plans, and the allocation-free table array.
// The kernels, and what they compute, are in zr_rsf_kernel.hpp.
#include <climits>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "zr_rsf_kernel.hpp"

namespace zr {
namespace {

using rsf::Fns;
using rsf::RsfArgs;
using rsf::RsfCommon;
using rsf::RsfWsArgs;
using rsf::kAnyPhase;
using rsf::kElemTile;

// Output block the vector tiles' writes are aligned to (bytes): tiles whose
// writes straddle 16 KiB blocks streamed 2-4% slower.
constexpr uintptr_t kOutBlock = 16384;

// Elements from the partition-side address `out` to the next kOutBlock
// boundary.
int64_t to_block(uintptr_t out, uintptr_t out_es) { return (int64_t)((kOutBlock - out % kOutBlock) % kOutBlock / out_es); }

// Head of a segment whose K rank runs start at byte addresses addr[r] and
// whose output starts at `out`: the offset of the first 128-byte line of
// rank j at or after the output's next kOutBlock boundary, with the
// kAnyPhase flag when the runs do not share one quad phase (the tiles then
// read the other ranks as aligned pairs).
int segment_head(const uintptr_t* addr, int K, int j, uintptr_t es, uintptr_t out, uintptr_t out_es) {
    const uintptr_t quad = 4 * es;
    bool same = true;
    for (int r = 1; r < K; ++r) same = same && (addr[r] - addr[0]) % quad == 0;
    const int64_t line = (int64_t)(128 / es);
    const int64_t to_line = (int64_t)(((128 - addr[j] % 128) % 128) / es);
    const int64_t b = to_block(out, out_es);
    const int h = (int)(b + ((to_line - b) % line + line) % line);
    return same ? h : (h | kAnyPhase);
}
static_assert(kOutBlock / 2 + 64 < (uintptr_t)kAnyPhase, "segment heads must stay below the flag bit");

// One (fragment, chunk) segment of the virtual bucket.
struct SegDesc {
    int m;       // entry
    int j;       // chunk
    int head;    // vector tiles start here (kAnyPhase: ranks in different quad phases); -1: element-wise
    int64_t tiles;
};

// Every entry's segments in order (entry ei's are [first[ei], first[ei+1])),
// with their heads and tile counts for vector tiles of T elements (-1 heads,
// element by element, only under ZR_FORCE_PATH=element).
template <typename TIn, typename TOut>
void segments_of(const RsfCommon& c, const FragEntry* entries, int n_entries, int64_t T,
                 std::vector<SegDesc>* segs, std::vector<int64_t>* first) {
    const int K = c.K;
    const int64_t C = c.C;
    segs->clear();
    first->assign(1, 0);
    for (int ei = 0; ei < n_entries; ++ei) {
        const FragEntry& f = entries[ei];
        const bool pad = f.ptr[0] == nullptr;
        const int j0 = (int)(f.off / C), j1 = (int)((f.off + f.n - 1) / C);
        for (int j = j0; j <= j1; ++j) {
            const int64_t jc = (int64_t)j * C;
            const int64_t lo = f.off > jc ? f.off : jc;
            const int64_t hi = (f.off + f.n) < jc + C ? (f.off + f.n) : jc + C;
            const int64_t len = hi - lo;
            const int q = ((j - c.shift) % K + K) % K;  // holder
            const uintptr_t o = (uintptr_t)c.out.p[q] + (uintptr_t)(lo - jc) * sizeof(TOut);
            int h;
            if (tuning().force_path == kPathElement) {
                h = -1;  // element-wise folds, forced
            } else if (pad) {
                // no input: align the partition side to its 16 KiB blocks
                h = (int)to_block(o, sizeof(TOut));
            } else {
                uintptr_t addr[kMaxRanks];
                for (int r = 0; r < K; ++r)
                    addr[r] = (uintptr_t)f.ptr[r] + (uintptr_t)(lo - f.off) * sizeof(TIn);
                h = segment_head(addr, K, j, sizeof(TIn), o, sizeof(TOut));
            }
            const int64_t hv = h < 0 ? h : (h & (kAnyPhase - 1));  // the head itself
            const int64_t hc = hv < len ? hv : len;
            const int64_t tiles = h < 0 ? (len + kElemTile - 1) / kElemTile
                                        : (hc + T - 1) / T + (len > hv ? (len - hv + T - 1) / T : 0);
            segs->push_back(SegDesc{ei, j, h, tiles});
        }
        first->push_back((int64_t)segs->size());
    }
}

// Cuts the entries into argument launches: each fills one argument block with
// up to kRsfEntriesPerLaunch fragments (and kRsfPtrsPerLaunch rank pointers),
// the padding entry if it comes next (it takes no pointers), and the segments
// they form with the chunks, keeping tile numbers within 32 bits.
void cut_args(const RsfCommon& c, const FragEntry* entries, int n_entries,
              const std::vector<SegDesc>& segs, const std::vector<int64_t>& first,
              std::vector<RsfArgs>* out) {
    const int K = c.K;
    const int max_entries = (kRsfPtrsPerLaunch / K) < kRsfEntriesPerLaunch ? (kRsfPtrsPerLaunch / K)
                                                                         : kRsfEntriesPerLaunch;
    RsfArgs a;
    std::memset(&a, 0, sizeof(a));
    a.c = c;
    a.c.pad_m = -1;
    int m = 0;
    int64_t tiles = 0;
    auto flush = [&]() {
        if (m == 0) return;
        a.tile0[a.nseg] = (int32_t)tiles;
        out->push_back(a);
        m = 0;
        tiles = 0;
        a.nseg = 0;
        a.c.pad_m = -1;
    };
    for (int ei = 0; ei < n_entries; ++ei) {
        const FragEntry& f = entries[ei];
        const bool pad = f.ptr[0] == nullptr;
        const int64_t s0 = first[ei], s1 = first[ei + 1];
        int64_t et = 0;
        for (int64_t s = s0; s < s1; ++s) et += segs[s].tiles;
        if (m == (pad ? max_entries + 1 : max_entries) || a.c.pad_m >= 0 ||
            a.nseg + (s1 - s0) > kRsfSegsPerLaunch || tiles + et > INT32_MAX / 2)
            flush();
        a.off[m] = f.off;
        a.n[m] = f.n;
        if (pad)
            a.c.pad_m = m;
        else
            for (int r = 0; r < K; ++r) a.ptr[m * K + r] = f.ptr[r];
        for (int64_t s = s0; s < s1; ++s) {
            const int d = a.nseg++;
            a.seg_m[d] = (uint8_t)m;
            a.seg_j[d] = (uint8_t)segs[s].j;
            a.seg_head[d] = (int16_t)segs[s].head;
            a.tile0[d] = (int32_t)tiles;
            tiles += segs[s].tiles;
        }
        ++m;
    }
    flush();
}

// The staged table's image for workspace `ws` (device addresses filled in).
void build_image(const RsfCommon& c, const FragEntry* entries, int n_entries,
                 const std::vector<SegDesc>& segs, uintptr_t ws, RsfWsArgs* wa, int64_t* tiles,
                 std::vector<uint8_t>* image) {
    const int K = c.K;
    const RsfLayout L(K, n_entries, (int64_t)segs.size());
    image->assign(L.bytes, 0);
    uint8_t* base = image->data();
    int64_t* tile0 = reinterpret_cast<int64_t*>(base + L.tile0);
    int32_t* sg = reinterpret_cast<int32_t*>(base + L.seg);
    int64_t* en = reinterpret_cast<int64_t*>(base + L.ent);
    uint64_t* pt = reinterpret_cast<uint64_t*>(base + L.ptr);
    *wa = RsfWsArgs{};
    wa->c = c;
    wa->c.pad_m = -1;
    for (int m = 0; m < n_entries; ++m) {
        en[2 * m] = entries[m].off;
        en[2 * m + 1] = entries[m].n;
        if (entries[m].ptr[0] == nullptr) wa->c.pad_m = m;
        for (int r = 0; r < K; ++r) pt[(size_t)m * K + r] = (uint64_t)(uintptr_t)entries[m].ptr[r];
    }
    int64_t t = 0;
    for (size_t s = 0; s < segs.size(); ++s) {
        tile0[s] = t;
        sg[3 * s] = segs[s].m;
        sg[3 * s + 1] = segs[s].j;
        sg[3 * s + 2] = segs[s].head;
        t += segs[s].tiles;
    }
    tile0[segs.size()] = t;
    *tiles = t;
    wa->tile0 = ws + L.tile0;
    wa->seg = ws + L.seg;
    wa->ent = ws + L.ent;
    wa->ptr = ws + L.ptr;
    wa->nseg = (int64_t)segs.size();
}

}  // namespace

struct RsfPlan {
    std::vector<RsfArgs> launches;  // argument launches, or
    bool staged = false;            // one launch over the table staged in the workspace
    RsfWsArgs wsa;
    int64_t ws_tiles = 0;
    std::vector<uint8_t> image;
    Fns fn{nullptr, nullptr};
};

RsfPlan* rsf_plan_build(int K, const FragEntry* entries, int n_entries, int64_t N, zr_dtype in_dt,
                        const MutPtrs& out, zr_dtype out_dt, int shift, int flags, zr_order order,
                        void* ws) {
    RsfPlan* plan = new (std::nothrow) RsfPlan();
    if (!plan) return nullptr;
    RsfCommon c;
    c.out = out;
    c.K = K;
    c.C = (N + K - 1) / K;
    c.shift = shift;
    c.accumulate = (flags & ZR_ACCUMULATE) ? 1 : 0;
    c.pad_m = -1;
    c.inv_k = 1.0f / (float)K;
    c.kf = (float)K;
    const bool pow2 = (K & (K - 1)) == 0;
    const int avg = !(flags & ZR_AVERAGE) ? 0 : (pow2 ? 1 : 2);
    const int ord = order == ZR_ORDER_FREE ? kFree : (order == ZR_ORDER_RING_WIRE ? kWire : kRing);
    // the tiles at full size decide the tile: launches that would give fewer
    // than two tiles per CU (ring order) use one slice per wave
    auto build = [&](auto tin, auto tout) {
        using TIn = decltype(tin);
        using TOut = decltype(tout);
        std::vector<SegDesc> segs;
        std::vector<int64_t> first;
        segments_of<TIn, TOut>(c, entries, n_entries, kRsTile<TIn, TOut>, &segs, &first);
        cut_args(c, entries, n_entries, segs, first, &plan->launches);
        plan->staged = ws != nullptr && plan->launches.size() > 1;
        int64_t most = 0;
        if (plan->staged) {
            for (const SegDesc& d : segs) most += d.tiles;
        } else {
            for (const RsfArgs& l : plan->launches) most = most > l.tile0[l.nseg] ? most : l.tile0[l.nseg];
        }
        const int fp = tuning().force_path;
        // fewer than two full tiles per CU for each eight ranks: one-slice tiles
        const int64_t k8 = (K + 7) / 8;
        const bool small = ord == kRing && (fp == kPathSmall || (fp != kPathLarge && most < 2LL * k8 * device_cu_count()));
        // ranks in different phases (a flag of the heads, whatever the tile)
        bool any = false;
        for (const SegDesc& d : segs) any = any || (d.head >= 0 && (d.head & kAnyPhase) != 0);
        // the free and generic wire kernels' tiles, and those of the kernels
        // for ranks in different phases, may hold fewer slices
        const bool narrow = any || rs_generic_narrow<TIn>(K, ord);
        const int64_t tile = small ? kRsTileOf<1>
                                   : (narrow ? kRsTileOf<kSlicesGeneric<TIn, TOut>> : kRsTile<TIn, TOut>);
        const bool retile = tile != kRsTile<TIn, TOut>;
        if (retile) segments_of<TIn, TOut>(c, entries, n_entries, tile, &segs, &first);
        if (plan->staged) {
            plan->launches.clear();
            build_image(c, entries, n_entries, segs, (uintptr_t)ws, &plan->wsa, &plan->ws_tiles, &plan->image);
        } else if (retile) {
            plan->launches.clear();
            cut_args(c, entries, n_entries, segs, first, &plan->launches);
        }
        plan->fn = rsf::pick_avg<TIn, TOut>(K, avg, ord, small, any);
    };
    try {
        if (in_dt == ZR_BF16 && out_dt == ZR_FP32)
            build(uint16_t{}, float{});
        else if (in_dt == ZR_BF16 && out_dt == ZR_BF16)
            build(uint16_t{}, uint16_t{});
        else if (in_dt == ZR_FP32 && out_dt == ZR_FP32)
            build(float{}, float{});
        else
            build(float{}, uint16_t{});
    } catch (...) {
        delete plan;
        return nullptr;
    }
    return plan;
}

size_t rsf_plan_table_bytes(const RsfPlan* plan) { return plan->staged ? plan->image.size() : 0; }
const void* rsf_plan_table_image(const RsfPlan* plan) { return plan->image.data(); }
int rsf_plan_launch_count(const RsfPlan* plan) {
    return plan->staged ? (plan->ws_tiles > 0 ? 1 : 0) : (int)plan->launches.size();
}

hipError_t rsf_plan_launch(const RsfPlan* plan, hipStream_t stream) {
    if (plan->staged) return plan->ws_tiles > 0 ? plan->fn.ws(plan->wsa, plan->ws_tiles, stream) : hipSuccess;
    for (const RsfArgs& a : plan->launches) {
        hipError_t e = plan->fn.args(a, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

void rsf_plan_free(RsfPlan* plan) { delete plan; }

// The table staging area of the entry point that allocates nothing: one
// array per GPU, held until the process ends. Host code never uses the name
// `scratch` as an address; it uses the device address looked up per device.
static __device__ __align__(256) unsigned char scratch[ZR_NOALLOC_TABLE_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace zr
