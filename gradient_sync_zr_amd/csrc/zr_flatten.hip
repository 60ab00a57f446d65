// IPG bucket flatten: fragmented gradients copied into one flat bucket per
// rank at running offsets, then the bucket's tail zero-filled up to the
// padded size ("DeepSpeed ZeRO-3 源码解析", 3.2 and 5.1: each grad lives at
// offset n_0 + ... + n_{p-1} of the flat buffer; 3.1: one large contiguous
// message instead of one per parameter).
//
// Every rank has the same fragment sizes, so a fragment is one entry: its
// bucket offset and size, shared by the ranks, and its K source pointers.
// Entry m owns K runs of tiles_per_rank[m] tiles, rank by rank. The table of
// entries rides in the kernel arguments when it fits one argument block: up
// to 32 entries' pointers (256 pointers, so 4 entries at K = 64), the zero
// padding in a spare slot after them (it has no source), and each entry's
// first tile; more entries go out as further launches (a block finds its
// entry by a uniform binary search over the first tiles). Given a workspace, a
// larger table is staged there and one launch copies every fragment (the
// bucket as one operation, section 3.1); the kernel reads it with scalar loads
// and finds a tile's entry with a wave-wide search. The grid has one block per
// tile of the launch, in order, so blocks stay balanced however unequal the
// fragments are, and the blocks in flight work on one compact window of
// memory (a persistent grid striding over the tiles ran 15-20% slower on a
// plain copy).
//
// A tile is 4 KiB of destination: lane l of wave w moves the 16-byte unit
// w*64 + l, so every store instruction of a wave covers 1 KiB contiguously;
// loads and stores are non-temporal (each byte is touched once). (At one
// block per tile 4 KiB tiles ran 8% faster than 8 or 16 KiB tiles.) Units
// are aligned to the destination, whose offsets inside a bucket are prefix
// sums of arbitrary sizes; a source in another 16-byte phase is read as
// aligned 16-byte blocks and realigned in registers, so every whole unit
// moves with 16-byte accesses; only a copy's partial first and last units go
// element by element.
#include <cstring>
#include <new>
#include <vector>

#include "zr_device.hpp"
#include "zr_internal.hpp"

namespace zr {
namespace {

// One 16-byte unit per lane: a tile is 4 KiB of destination.
constexpr int64_t kFlatTileBytes = (int64_t)kThreads * 16;

// Entry slots: fragments with source pointers, plus one for the padding.
constexpr int kFlatSlots = kFlatEntriesPerLaunch + 1;

// Fields every launch carries, whichever table it reads.
struct FlatCommon {
    MutPtrs bucket;  // rank r's bucket
    int K;
    int pad_m;       // the padding entry (writes zeros), -1: none
};

// A launch whose table rides in its kernel arguments.
struct FlatArgs {
    FlatCommon c;
    const void* src[kFlatPtrsPerLaunch];  // entry-major: src[m * K + r]
    int64_t off[kFlatSlots];               // bucket offset of entry m (elements)
    int64_t n[kFlatSlots];                 // elements of entry m
    int32_t tile0[kFlatSlots + 1];         // first tile of entry m; tile0[nent] = all tiles
    int32_t tpr[kFlatSlots];               // tiles of entry m per rank
    int nent;
};
static_assert(sizeof(FlatArgs) <= 4096, "flatten arguments exceed 4 KB");

// A launch whose table is staged in a workspace (the layout of flatten_table_bytes).
struct FlatWsArgs {
    FlatCommon c;
    uint64_t tile0;  // int64_t[nent + 1]: first tile of entry m; tile0[nent] = all tiles
    uint64_t tpr;    // int64_t[nent]: tiles of entry m per rank
    uint64_t ent;    // int64_t[2 * nent]: bucket offset and size of entry m at 2m
    uint64_t src;    // const void*[K * nent], entry-major (null for the padding entry)
    int64_t nent;
};

struct FlatEnt {
    int64_t off, n, tpr;
};

struct FlatArgTable {
    using Index = int;  // argument launches keep tile numbers within 32 bits
    const FlatArgs& a;
    __device__ __forceinline__ int total() const { return a.tile0[a.nent]; }
    // the last m with tile0[m] <= t, by a uniform binary search on scalar
    // loads of the arguments (a wave-wide search on vector loads of them ran
    // the 4 KiB tiles 10% slower: it puts an extra vector-memory round trip
    // ahead of every tile's one load)
    __device__ __forceinline__ int find(int, int t) const {
        int lo = 0, hi = a.nent;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.tile0[mid] <= t)
                lo = mid;
            else
                hi = mid;
        }
        return lo;
    }
    __device__ __forceinline__ int first(int m) const { return a.tile0[m]; }
    __device__ __forceinline__ FlatEnt ent(int m) const { return {a.off[m], a.n[m], a.tpr[m]}; }
    __device__ __forceinline__ const void* src(int m, int K, int r) const { return a.src[m * K + r]; }
};

struct FlatWsTable {
    using Index = int64_t;
    cptr<int64_t> tile0, tpr, en;
    cptr<const void*> srcs;
    int64_t nent;
    __device__ __forceinline__ explicit FlatWsTable(const FlatWsArgs& a)
        : tile0(table_at<int64_t>(a.tile0)), tpr(table_at<int64_t>(a.tpr)), en(table_at<int64_t>(a.ent)),
          srcs(table_at<const void*>(a.src)), nent(a.nent) {}
    __device__ __forceinline__ int64_t total() const { return tile0[nent]; }
    __device__ __forceinline__ int64_t find(int64_t, int64_t t) const { return find_slot64(tile0, nent, t); }
    __device__ __forceinline__ int64_t first(int64_t m) const { return tile0[m]; }
    __device__ __forceinline__ FlatEnt ent(int64_t m) const { return {en[2 * m], en[2 * m + 1], tpr[m]}; }
    __device__ __forceinline__ const void* src(int64_t m, int K, int r) const { return srcs[m * K + r]; }
};

// Units are 16-byte blocks of the destination, counted from the block that
// holds the copy's first byte. A unit wholly inside the copy is stored as
// one aligned 16-byte store; its 16 source bytes come from one aligned load
// when source and destination share their phase within 16 bytes, else from
// the two aligned 16-byte blocks that hold them (both hold bytes of the
// fragment, so neither read leaves its pages), joined in registers. The
// first and last units, when partial, copy element by element (all loads of
// a lane before its stores).
template <typename T, typename Tab>
__device__ __forceinline__ void flatten_body(const FlatCommon& c, const Tab& tab) {
    constexpr int per = 16 / sizeof(T);  // elements per 16-byte unit
    using Index = typename Tab::Index;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const Index total = tab.total();
    Index m = 0;
    for (Index t = blockIdx.x; t < total; t += gridDim.x) {
        m = tab.find(m, t);
        const FlatEnt fe = tab.ent(m);
        const Index tt = t - tab.first(m);
        const int r = (int)(tt / (Index)fe.tpr);  // the entry's tiles run rank by rank
        const int64_t lt = tt - (int64_t)r * fe.tpr;
        const T* src = m == c.pad_m ? nullptr : static_cast<const T*>(tab.src(m, c.K, r));
        T* dst = static_cast<T*>(c.bucket.p[r]) + fe.off;
        const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (uintptr_t)fe.n * sizeof(T);
        const uintptr_t ub = (d0 & ~(uintptr_t)15) +
                             16 * (uintptr_t)(lt * (kFlatTileBytes / 16) + wave * 64 + lane);
        if (ub >= d0 && ub + 16 <= d1) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (src) {
                const uintptr_t sb = (uintptr_t)src + (ub - d0);
                const uint32_t sig = (uint32_t)(sb & 15);
                const u32x4* a = reinterpret_cast<const u32x4*>(sb & ~(uintptr_t)15);
                if (sig == 0) {
                    v = ld<true>(a);
                } else {
                    const u32x4 lo = ld<true>(a), hi = ld<true>(a + 1);
                    v = shift16(lo, hi, sig);
                }
            }
            st<true>(reinterpret_cast<u32x4*>(ub), v);
        } else if (ub < d1 && ub + 16 > d0) {
            const int64_t e0 = (int64_t)(((ub > d0 ? ub : d0) - d0) / sizeof(T));
            const int64_t e1 = (int64_t)(((ub + 16 < d1 ? ub + 16 : d1) - d0) / sizeof(T));
            T ev[per];
#pragma unroll
            for (int e = 0; e < per; ++e)
                if (e0 + e < e1) ev[e] = src ? src[e0 + e] : T(0);
#pragma unroll
            for (int e = 0; e < per; ++e)
                if (e0 + e < e1) dst[e0 + e] = ev[e];
        }
    }
}

template <typename T>
__global__ void __launch_bounds__(kThreads) flatten_kernel(const FlatArgs a) {
    flatten_body<T>(a.c, FlatArgTable{a});
}

template <typename T>
__global__ void __launch_bounds__(kThreads) flatten_ws_kernel(const FlatWsArgs a) {
    flatten_body<T>(a.c, FlatWsTable(a));
}

int64_t tiles_of(int64_t bytes, int64_t tile) { return (bytes + tile - 1) / tile; }

// Tiles per rank of a copy of n elements to bucket offset `off` (elements):
// its units start at the 16-byte block holding its first byte on every rank,
// so a rank whose copy starts b bytes into a block needs room for b + n*es.
int64_t tiles_per_rank(const MutPtrs& buckets, int K, int64_t off, int64_t n, int elem_bytes) {
    int64_t lead = 0;
    for (int r = 0; r < K; ++r) {
        const int64_t b = (int64_t)(((uintptr_t)buckets.p[r] + (uintptr_t)off * elem_bytes) & 15);
        lead = b > lead ? b : lead;
    }
    return tiles_of(lead + n * elem_bytes, kFlatTileBytes);
}

// Cuts the entries into argument launches of at most 32 fragments (256
// source pointers) plus the padding entry if it comes next, and about 2^29
// tiles; an entry of more than 2^28 / K tiles per rank is cut into pieces of
// that many first, so tile numbers fit in 32 bits.
void cut_args(const FlatCommon& c, const FragEntry* entries, int n_entries, int elem_bytes,
              std::vector<FlatArgs>* out) {
    const int K = c.K;
    const int max_entries = (kFlatPtrsPerLaunch / K) < kFlatEntriesPerLaunch ? (kFlatPtrsPerLaunch / K)
                                                                           : kFlatEntriesPerLaunch;
    const int64_t piece = ((1LL << 28) / K) * (kFlatTileBytes / elem_bytes);  // elements
    FlatArgs a;
    std::memset(&a, 0, sizeof(a));
    a.c = c;
    a.c.pad_m = -1;
    int count = 0;
    int64_t tiles = 0;
    auto flush = [&]() {
        if (count == 0) return;
        a.tile0[count] = (int32_t)tiles;
        a.nent = count;
        if (tiles > 0) out->push_back(a);
        count = 0;
        tiles = 0;
        a.c.pad_m = -1;
    };
    for (int i = 0; i < n_entries; ++i) {
        const FragEntry& f = entries[i];
        const bool is_pad = f.ptr[0] == nullptr;
        for (int64_t o = 0; o < f.n; o += piece) {
            const int64_t pn = f.n - o < piece ? f.n - o : piece;
            const int64_t tpr = tiles_per_rank(c.bucket, K, f.off + o, pn, elem_bytes);
            if (count == (is_pad ? max_entries + 1 : max_entries) || a.c.pad_m >= 0 ||
                tiles + (int64_t)K * tpr > (1LL << 29))
                flush();
            a.off[count] = f.off + o;
            a.n[count] = pn;
            if (is_pad)
                a.c.pad_m = count;
            else
                for (int r = 0; r < K; ++r) a.src[count * K + r] = static_cast<const char*>(f.ptr[r]) + o * elem_bytes;
            a.tpr[count] = (int32_t)tpr;
            a.tile0[count] = (int32_t)tiles;
            tiles += (int64_t)K * tpr;
            ++count;
        }
    }
    flush();
}

}  // namespace

struct FlatPlan {
    std::vector<FlatArgs> launches;  // argument launches, or
    bool staged = false;             // one launch over the table staged in the workspace
    FlatWsArgs wsa;
    int64_t ws_tiles = 0;
    std::vector<uint8_t> image;
    int elem_bytes = 2;
};

FlatPlan* flat_plan_build(int K, const FragEntry* entries, int n_entries, const MutPtrs& buckets,
                          int elem_bytes, void* ws) {
    FlatPlan* plan = new (std::nothrow) FlatPlan();
    if (!plan) return nullptr;
    try {
        FlatCommon c;
        c.bucket = buckets;
        c.K = K;
        c.pad_m = -1;
        plan->elem_bytes = elem_bytes;
        cut_args(c, entries, n_entries, elem_bytes, &plan->launches);
        if (ws != nullptr && plan->launches.size() > 1) {
            plan->launches.clear();
            plan->staged = true;
            const FlatLayout L(K, n_entries);
            plan->image.assign(L.bytes, 0);
            uint8_t* base = plan->image.data();
            int64_t* tile0 = reinterpret_cast<int64_t*>(base + L.tile0);
            int64_t* tpr = reinterpret_cast<int64_t*>(base + L.tpr);
            int64_t* en = reinterpret_cast<int64_t*>(base + L.ent);
            uint64_t* src = reinterpret_cast<uint64_t*>(base + L.src);
            int64_t tiles = 0;
            for (int m = 0; m < n_entries; ++m) {
                const FragEntry& f = entries[m];
                if (f.ptr[0] == nullptr) c.pad_m = m;
                tile0[m] = tiles;
                tpr[m] = tiles_per_rank(buckets, K, f.off, f.n, elem_bytes);
                en[2 * m] = f.off;
                en[2 * m + 1] = f.n;
                for (int r = 0; r < K; ++r) src[(size_t)m * K + r] = (uint64_t)(uintptr_t)f.ptr[r];
                tiles += (int64_t)K * tpr[m];
            }
            tile0[n_entries] = tiles;
            const uintptr_t w = (uintptr_t)ws;
            plan->wsa = FlatWsArgs{};
            plan->wsa.c = c;
            plan->wsa.tile0 = w + L.tile0;
            plan->wsa.tpr = w + L.tpr;
            plan->wsa.ent = w + L.ent;
            plan->wsa.src = w + L.src;
            plan->wsa.nent = n_entries;
            plan->ws_tiles = tiles;
        }
    } catch (...) {
        delete plan;
        return nullptr;
    }
    return plan;
}

size_t flat_plan_table_bytes(const FlatPlan* plan) { return plan->staged ? plan->image.size() : 0; }
const void* flat_plan_table_image(const FlatPlan* plan) { return plan->image.data(); }
int flat_plan_launch_count(const FlatPlan* plan) {
    return plan->staged ? (plan->ws_tiles > 0 ? 1 : 0) : (int)plan->launches.size();
}

hipError_t flat_plan_launch(const FlatPlan* plan, hipStream_t stream) {
    if (plan->staged) {
        if (plan->ws_tiles == 0) return hipSuccess;
        const int gx = grid_for(plan->ws_tiles);  // one block per tile, striding beyond the cap
        if (plan->elem_bytes == 2)
            hipLaunchKernelGGL((flatten_ws_kernel<uint16_t>), dim3(gx), dim3(kThreads), 0, stream, plan->wsa);
        else
            hipLaunchKernelGGL((flatten_ws_kernel<uint32_t>), dim3(gx), dim3(kThreads), 0, stream, plan->wsa);
        return hipGetLastError();
    }
    for (const FlatArgs& a : plan->launches) {
        const int gx = grid_for(a.tile0[a.nent]);  // one block per tile
        if (plan->elem_bytes == 2)
            hipLaunchKernelGGL((flatten_kernel<uint16_t>), dim3(gx), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((flatten_kernel<uint32_t>), dim3(gx), dim3(kThreads), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

void flat_plan_free(FlatPlan* plan) { delete plan; }

}  // namespace zr
