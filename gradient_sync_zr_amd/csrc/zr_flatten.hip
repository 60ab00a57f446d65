// IPG bucket flatten: fragmented gradients copied into one flat bucket per
// rank at running offsets, then the bucket's tail zero-filled up to the
// padded size ("DeepSpeed ZeRO-3 源码解析", 3.2 and 5.1: each grad lives at
// offset n_0 + ... + n_{p-1} of the flat buffer; 3.1: one large contiguous
// message instead of one per parameter).
//
// Every rank has the same fragment sizes, so a fragment is one entry: its
// bucket offset and size, shared by the ranks, and its K source pointers. A
// launch carries up to 32 entries' pointers (256 pointers, so 4 entries at
// K = 64), the zero padding in a spare slot after them (it has no source),
// the K bucket bases and each entry's first tile, all in its kernel
// arguments: no device descriptor table, no staging copy. Entry m owns K
// runs of tiles_per_rank[m] tiles, rank by rank. The grid has one block per
// tile of the launch, in order, so blocks stay balanced however unequal the
// fragments are, and the blocks in flight work on one compact window of
// memory (a persistent grid striding over the tiles ran 15-20% slower on a
// plain copy).
//
// A tile is 4 KiB of destination: lane l of wave w moves the 16-byte unit
// w*64 + l, so every load and store instruction of a wave covers 1 KiB
// contiguously; loads and stores are non-temporal (each byte is touched
// once). (At one block per tile a plain copy ran 10-15% faster with 4 KiB
// tiles than with 16 KiB tiles of four units per lane; in the flatten the
// two sizes measure the same, and one size needs no small-launch mode.) A copy whose source
// and destination both start 16-byte aligned moves whole units; its last
// partial unit, and every unit of a copy that is not aligned so (possible
// inside a bucket, where offsets are prefix sums of arbitrary sizes), copies
// element by element.
#include "zr_device.hpp"
#include "zr_internal.hpp"

namespace zr {
namespace {

// 16-byte units per lane, and the tile they make.
constexpr int kUnits = 1;
constexpr int64_t kFlatTileBytes = (int64_t)kThreads * 16 * kUnits;

// Entry slots: fragments with source pointers, plus one for the padding.
constexpr int kFlatSlots = kFlatEntriesPerLaunch + 1;

struct FlatArgs {
    const void* src[kFlatPtrsPerLaunch];  // entry-major: src[m * K + r]
    void* bucket[kMaxRanks];               // rank r's bucket
    int64_t off[kFlatSlots];               // bucket offset of entry m (elements)
    int64_t n[kFlatSlots];                 // elements of entry m
    int32_t tile0[kFlatSlots + 1];         // first tile of entry m; tile0[nent] = all tiles
    int32_t tpr[kFlatSlots];               // tiles of entry m per rank
    int K, nent, pad_m;                    // pad_m: the padding entry (writes zeros), -1: none
};
static_assert(sizeof(FlatArgs) <= 4096, "flatten arguments exceed 4 KB");

template <typename T>
__global__ void __launch_bounds__(kThreads) flatten_kernel(const FlatArgs a) {
    constexpr int per = 16 / sizeof(T);  // elements per 16-byte unit
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int total = a.tile0[a.nent];
    int m = 0;
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        m = find_slot(a.tile0, a.nent, m, t);  // a block's tiles only grow: entries in order
        const int tt = t - a.tile0[m];
        const int r = tt / a.tpr[m];            // the entry's tiles run rank by rank
        const int64_t lt = tt - (int64_t)r * a.tpr[m];
        const int64_t n = a.n[m];
        const T* src = m == a.pad_m ? nullptr : static_cast<const T*>(a.src[m * a.K + r]);
        T* dst = static_cast<T*>(a.bucket[r]) + a.off[m];
        const bool vec = ((((uintptr_t)dst) & 15) == 0) && (src == nullptr || (((uintptr_t)src) & 15) == 0);
        const int64_t u0 = lt * (kFlatTileBytes / 16) + wave * 64 * kUnits + lane;  // first unit
        if (vec && (u0 + 64 * (kUnits - 1) + 1) * per <= n) {
            // every unit of this lane is whole
            u32x4 v[kUnits];
#pragma unroll
            for (int k = 0; k < kUnits; ++k)
                v[k] = src ? ld<true>(reinterpret_cast<const u32x4*>(src + (u0 + 64 * k) * per))
                           : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < kUnits; ++k)
                st<true>(reinterpret_cast<u32x4*>(dst + (u0 + 64 * k) * per), v[k]);
            continue;
        }
        // some unit of this lane is partial or unaligned: every load is issued
        // before the first store (a store may not overtake the loads, so the
        // lane waits on one memory latency, not one per element)
        u32x4 vv[kUnits];
        T ev[kUnits][per];
        int cnt[kUnits];
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const int64_t e0 = (u0 + 64 * k) * per;
            cnt[k] = e0 >= n ? 0 : (int)((n - e0) < per ? (n - e0) : per);
            if (vec && cnt[k] == per) {
                vv[k] = src ? ld<true>(reinterpret_cast<const u32x4*>(src + e0)) : u32x4{0u, 0u, 0u, 0u};
            } else {
#pragma unroll
                for (int e = 0; e < per; ++e)
                    if (e < cnt[k]) ev[k][e] = src ? src[e0 + e] : T(0);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const int64_t e0 = (u0 + 64 * k) * per;
            if (vec && cnt[k] == per) {
                st<true>(reinterpret_cast<u32x4*>(dst + e0), vv[k]);
            } else {
#pragma unroll
                for (int e = 0; e < per; ++e)
                    if (e < cnt[k]) dst[e0 + e] = ev[k][e];
            }
        }
    }
}

template <typename T>
hipError_t launch_batch(const FlatArgs& a, hipStream_t stream) {
    const int64_t tiles = a.tile0[a.nent];
    const int gx = grid_for(tiles);  // one block per tile
    hipLaunchKernelGGL((flatten_kernel<T>), dim3(gx), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

int64_t tiles_of(int64_t bytes, int64_t tile) { return (bytes + tile - 1) / tile; }

}  // namespace

// Entries go out in launches of at most 32 fragments (256 source pointers)
// plus the padding entry if it comes next, and about 2^29 tiles; a larger
// entry has already been split by the caller, so tile numbers fit in 32 bits.
hipError_t launch_flatten(int K, const FragEntry* entries, int n_entries, const MutPtrs& buckets,
                          int elem_bytes, hipStream_t stream) {
    const int max_entries = (kFlatPtrsPerLaunch / K) < kFlatEntriesPerLaunch ? (kFlatPtrsPerLaunch / K)
                                                                           : kFlatEntriesPerLaunch;
    FlatArgs a;
    a.K = K;
    for (int r = 0; r < K; ++r) a.bucket[r] = buckets.p[r];
    int first = 0, count = 0, pad = -1;
    int64_t batch = 0;  // tiles of the batch
    auto flush = [&]() -> hipError_t {
        if (count == 0) return hipSuccess;
        const int64_t tile = kFlatTileBytes;
        int64_t tiles = 0;
        for (int i = 0; i < count; ++i) {
            const FragEntry& f = entries[first + i];
            a.off[i] = f.off;
            a.n[i] = f.n;
            if (i != pad)
                for (int r = 0; r < K; ++r) a.src[i * K + r] = f.ptr[r];
            a.tpr[i] = (int32_t)tiles_of(f.n * elem_bytes, tile);
            a.tile0[i] = (int32_t)tiles;
            tiles += (int64_t)K * a.tpr[i];
        }
        a.tile0[count] = (int32_t)tiles;
        a.nent = count;
        a.pad_m = pad;
        hipError_t e = hipSuccess;
        if (tiles > 0)
            e = elem_bytes == 2 ? launch_batch<uint16_t>(a, stream) : launch_batch<uint32_t>(a, stream);
        first += count;
        count = 0;
        pad = -1;
        batch = 0;
        return e;
    };
    for (int i = 0; i < n_entries; ++i) {
        const bool is_pad = entries[i].ptr[0] == nullptr;
        if (count == (is_pad ? max_entries + 1 : max_entries) || pad >= 0 || batch > (1LL << 28)) {
            hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
        if (is_pad) pad = count;
        batch += (int64_t)K * tiles_of(entries[i].n * elem_bytes, kFlatTileBytes);
        ++count;
    }
    return flush();
}

}  // namespace zr
