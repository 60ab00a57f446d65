// All-gather of sharded tensors into K full copies.
//
// ZeRO-3 keeps each parameter as 1/K shards and gathers the full tensor
// before use ("DeepSpeed ZeRO-3 源码解析", sections 1 and 2.1); the ring's
// second phase forwards each reduced chunk around the ring, receivers
// overwriting their copy ("图解 Ring All-Reduce", Phase 2). On one device the
// forwarding collapses to: chunk j of the full tensor is shard
// (j - shift) mod K, copied to every rank's full buffer.
//
// Grid: one block per tile of the launch. The tiles of a segment (one
// tensor) are its (chunk, tile) pairs, chunk by chunk, and the segments'
// tiles follow each other, so blocks stay balanced however unequal the
// tensors are; a block finds its segment by a uniform binary search over the
// segments' first tiles. The segment table rides in the kernel arguments, 32
// segments per launch; given a workspace, any number of segments go out as
// one launch that reads a table staged there (scalar loads, wave-wide
// search). (A persistent grid striding over the tiles ran
// 10-15% slower.) A tile writes 16 KiB to every full buffer in 16-byte units
// (8 bf16 or 4 fp32 elements): each lane loads kAgSub units of the shard, all
// before its first store, and stores each to all K full buffers, so each
// shard byte is read once and written K times. Lane l of a wave takes unit l
// of each 1 KiB span, so every store instruction writes one contiguous 1 KiB.
// (Tiles of 16 KiB per destination ran 1% faster than tiles of 4, 8 or
// 32 KiB. With 32-byte fp32 groups per lane, each store instruction covered
// its span at half density and fp32 gathers ran at 2.0-2.8 TB/s.) A chunk's
// units are aligned to its destination, whose start full_off + j*C may fall
// anywhere within 16 bytes (full_off is a running sum of tensor sizes); when
// the source is in another phase, each unit is read as the two aligned
// 16-byte blocks holding it and shifted into place in registers, so every
// whole unit moves with 16-byte loads and stores (element-by-element copies
// of such chunks ran 4.5x slower). The shards may sit at any phase (a chunk
// reads one shard). When the full buffers' phases differ, every destination
// has its own grid: the block stages the tile's source bytes in LDS once
// (aligned 16-byte loads) and each destination reads its units from there,
// shifted for its own phase (element-by-element copies of such gathers ran
// 5-7x slower). Only a chunk's partial first and last units copy element by
// element.
#include <vector>

#include "zr_device.hpp"
#include "zr_internal.hpp"

namespace zr {
namespace {

struct AgSeg {
    int64_t shard_off, full_off, numel, C;
    uint64_t vec_mask;  // bit j: chunk j moves whole units with 16-byte accesses
    int tiles_per_chunk;
    int pad_;
};
static_assert(sizeof(AgSeg) == kAgSegBytes, "staged all-gather records are kAgSegBytes each");

// Fields every launch carries, whichever table it reads.
struct AgCommon {
    ConstPtrs shards;
    MutPtrs fulls;
    int K, shift;
    int fphase;  // elements from the full buffers' common 16-byte phase (all equal when vec_mask is set)
};

// A launch whose segment table rides in its kernel arguments.
struct AgArgs {
    AgCommon c;
    AgSeg seg[kAgSegsPerLaunch];
    int64_t unit0[kAgSegsPerLaunch + 1];  // first tile of segment s; unit0[nseg] = all tiles
    int nseg;
};
static_assert(sizeof(AgArgs) <= 4096, "all-gather arguments exceed 4 KB");

// A launch whose table is staged in a workspace (the layout of ag_table_bytes).
struct AgWsArgs {
    AgCommon c;
    uint64_t unit0;  // int64_t[nseg + 1]
    uint64_t seg;    // AgSeg[nseg]
    int64_t nseg;
};

struct AgArgTable {
    const AgArgs& a;
    __device__ __forceinline__ int64_t total() const { return a.unit0[a.nseg]; }
    // the last s with unit0[s] <= u (uniform binary search)
    __device__ __forceinline__ int64_t find(int64_t u) const {
        int s = 0;
        for (int hi = a.nseg; hi - s > 1;) {
            const int mid = (s + hi) >> 1;
            if (a.unit0[mid] <= u)
                s = mid;
            else
                hi = mid;
        }
        return s;
    }
    __device__ __forceinline__ int64_t first(int64_t s) const { return a.unit0[s]; }
    __device__ __forceinline__ AgSeg seg(int64_t s) const { return a.seg[s]; }
};

struct AgWsTable {
    cptr<int64_t> unit0;
    cptr<AgSeg> segs;
    int64_t nseg;
    __device__ __forceinline__ explicit AgWsTable(const AgWsArgs& a)
        : unit0(table_at<int64_t>(a.unit0)), segs(table_at<AgSeg>(a.seg)), nseg(a.nseg) {}
    __device__ __forceinline__ int64_t total() const { return unit0[nseg]; }
    __device__ __forceinline__ int64_t find(int64_t u) const { return find_slot64(unit0, nseg, u); }
    __device__ __forceinline__ int64_t first(int64_t s) const { return unit0[s]; }
    __device__ __forceinline__ AgSeg seg(int64_t s) const {
        const cptr<AgSeg> p = segs + s;  // field by field: the record lives in the constant space
        AgSeg r;
        r.shard_off = p->shard_off;
        r.full_off = p->full_off;
        r.numel = p->numel;
        r.C = p->C;
        r.vec_mask = p->vec_mask;
        r.tiles_per_chunk = p->tiles_per_chunk;
        r.pad_ = 0;
        return r;
    }
};

// 16-byte units per lane in one tile (16 KiB per destination), the elements
// of a unit, and the elements of a tile.
constexpr int kAgSub = 16384 / (kThreads * 16);
template <typename T>
constexpr int kAgUnit = 16 / (int)sizeof(T);
template <typename T>
constexpr int64_t kAgTile = (int64_t)kAgSub * kThreads * kAgUnit<T>;

// The 16 bytes at p, which need only be element aligned: one aligned load,
// or the two aligned 16-byte blocks that hold them (each holds at least one
// of their bytes, so no read leaves their pages) joined in registers. The
// phase p & 15 must be uniform over the wave.
template <bool NT>
__device__ __forceinline__ u32x4 load16_any(const void* p) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t sig = (uint32_t)(a & 15);
    const u32x4* b = reinterpret_cast<const u32x4*>(a & ~(uintptr_t)15);
    if (sig == 0) return ld<NT>(b);
    return shift16(ld<NT>(b), ld<NT>(b + 1), sig);
}

template <typename T, int KS, bool NT, typename Tab>
__device__ __forceinline__ void ag_body(const AgCommon& a, const Tab& tab) {
    constexpr int SUB = kAgSub;
    constexpr int E = kAgUnit<T>;
    const int K = KS > 0 ? KS : a.K;
    const int64_t total = tab.total();
    for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
        // the tile's segment: the last s with unit0[s] <= u (uniform)
        const int64_t s = tab.find(u);
        const AgSeg sg = tab.seg(s);
        const int ul = (int)(u - tab.first(s));  // < K * tiles_per_chunk <= 2^29: 32-bit division
        const int j = ul / sg.tiles_per_chunk;
        const int t = ul - j * sg.tiles_per_chunk;
        int holder = j - a.shift;
        if (holder < 0) holder += K;
        const bool vec_chunk = (sg.vec_mask >> j) & 1ull;
        const T* shard = static_cast<const T*>(a.shards.p[holder]) + sg.shard_off;
        const int64_t dst0 = sg.full_off + (int64_t)j * sg.C;  // the chunk's start in every full buffer
        int64_t len = sg.numel - (int64_t)j * sg.C;            // its elements (<= 0: none)
        if (len > sg.C) len = sg.C;
        // unit k of this lane covers chunk offsets [x, x + E) with
        // x = ((t * SUB + k) * kThreads + tid) * E - lead: units start on the
        // destination's 16-byte grid
        const int64_t lead = vec_chunk ? ((a.fphase + dst0) & (E - 1)) : 0;
        u32x4 v[SUB];
        bool whole[SUB];
#pragma unroll
        for (int k = 0; k < SUB; ++k) {
            const int64_t x = (((int64_t)t * SUB + k) * kThreads + threadIdx.x) * E - lead;
            whole[k] = vec_chunk && x >= 0 && x + E <= len;
            if (whole[k]) v[k] = load16_any<NT>(shard + x);
        }
#pragma unroll
        for (int k = 0; k < SUB; ++k) {
            const int64_t x = (((int64_t)t * SUB + k) * kThreads + threadIdx.x) * E - lead;
            const int64_t dst_off = dst0 + x;
            if (whole[k]) {
                if constexpr (KS > 0) {
#pragma unroll
                    for (int r = 0; r < KS; ++r) st<NT>(reinterpret_cast<u32x4*>(static_cast<T*>(a.fulls.p[r]) + dst_off), v[k]);
                } else {
                    for (int r = 0; r < K; ++r) st<NT>(reinterpret_cast<u32x4*>(static_cast<T*>(a.fulls.p[r]) + dst_off), v[k]);
                }
            } else if (x < len && x + E > 0) {
                const int64_t e0 = x > 0 ? x : 0;
                const int64_t e1 = x + E < len ? x + E : len;
                for (int64_t e = e0; e < e1; ++e) {
                    const T val = shard[e];
                    for (int r = 0; r < K; ++r) static_cast<T*>(a.fulls.p[r])[dst0 + e] = val;
                }
            }
        }
    }
}

// The same tiles when the full buffers sit in different 16-byte phases.
// Destination r's units start on its own grid, lead_r = (its chunk start's
// element index) mod 16 / sizeof(T) elements before the chunk's offsets, so
// tile t covers chunk offsets [t tile - lead_r, (t+1) tile - lead_r) of it.
// The block stages the source elements every destination's tile t needs,
// [t tile - 16 / sizeof(T) + 1, (t+1) tile) within the chunk, as the aligned
// 16-byte blocks of the shard that hold them; a destination's whole unit is
// then one of those blocks, or two shifted into place.
template <typename T, bool NT, typename Tab>
__device__ __forceinline__ void ag_body_any(const AgCommon& a, const Tab& tab) {
    constexpr int SUB = kAgSub;
    constexpr int E = kAgUnit<T>;
    constexpr int64_t TILE = kAgTile<T>;
    constexpr int kBlocks = (int)(TILE * sizeof(T) / 16) + 2;  // 16-byte blocks a tile's span can touch
    __shared__ u32x4 stage[kBlocks];
    const int K = a.K;
    const int64_t total = tab.total();
    for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
        const int64_t s = tab.find(u);
        const AgSeg sg = tab.seg(s);
        const int ul = (int)(u - tab.first(s));
        const int j = ul / sg.tiles_per_chunk;
        const int t = ul - j * sg.tiles_per_chunk;
        int holder = j - a.shift;
        if (holder < 0) holder += K;
        const T* shard = static_cast<const T*>(a.shards.p[holder]) + sg.shard_off;
        const int64_t dst0 = sg.full_off + (int64_t)j * sg.C;
        int64_t len = sg.numel - (int64_t)j * sg.C;
        if (len > sg.C) len = sg.C;
        int64_t xs = (int64_t)t * TILE - (E - 1), xe = (int64_t)(t + 1) * TILE;
        xs = xs > 0 ? xs : 0;
        xe = xe < len ? xe : len;
        if (xs >= xe) continue;  // uniform: no element of this chunk in the tile
        const uintptr_t base = (uintptr_t)(shard + xs) & ~(uintptr_t)15;
        const int nb = (int)(((uintptr_t)(shard + xe) - base + 15) / 16);  // <= kBlocks
        for (int i = threadIdx.x; i < nb; i += kThreads) stage[i] = ld<NT>(reinterpret_cast<const u32x4*>(base) + i);
        __syncthreads();
        for (int r = 0; r < K; ++r) {
            T* full = static_cast<T*>(a.fulls.p[r]) + dst0;
            const int64_t lead = (int64_t)(((uintptr_t)full / sizeof(T)) & (E - 1));
#pragma unroll
            for (int k = 0; k < SUB; ++k) {
                const int64_t x = (((int64_t)t * SUB + k) * kThreads + threadIdx.x) * E - lead;
                if (x >= 0 && x + E <= len) {
                    // [x, x + E) lies in [xs, xe): its bytes are staged; a
                    // block past the unit's last byte is never read (at the
                    // span's end it lies beyond what was staged)
                    const uintptr_t off = (uintptr_t)(shard + x) - base;
                    const int blk = (int)(off / 16);
                    const uint32_t sig = (uint32_t)(off & 15);  // uniform: lanes step by whole units
                    u32x4 v;
                    if (sig == 0)
                        v = stage[blk];
                    else
                        v = shift16(stage[blk], stage[blk + 1], sig);
                    st<NT>(reinterpret_cast<u32x4*>(full + x), v);
                } else if (x < len && x + E > 0) {
                    const int64_t e0 = x > 0 ? x : 0;
                    const int64_t e1 = x + E < len ? x + E : len;
                    for (int64_t e = e0; e < e1; ++e) full[e] = shard[e];
                }
            }
        }
        __syncthreads();  // the stage is read before the next tile fills it
    }
}

template <typename T, int KS, bool NT, bool ANY>
__global__ void __launch_bounds__(kThreads) ag_kernel(const AgArgs a) {
    if constexpr (ANY)
        ag_body_any<T, NT>(a.c, AgArgTable{a});
    else
        ag_body<T, KS, NT>(a.c, AgArgTable{a});
}

template <typename T, int KS, bool NT, bool ANY>
__global__ void __launch_bounds__(kThreads) ag_ws_kernel(const AgWsArgs a) {
    if constexpr (ANY)
        ag_body_any<T, NT>(a.c, AgWsTable(a));
    else
        ag_body<T, KS, NT>(a.c, AgWsTable(a));
}

template <typename T, int KS, bool NT, bool ANY>
hipError_t launch_t(const AgArgs& a, hipStream_t stream) {
    const int gx = grid_for(a.unit0[a.nseg]);  // one block per tile
    hipLaunchKernelGGL((ag_kernel<T, KS, NT, ANY>), dim3(gx), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int KS, bool NT, bool ANY>
hipError_t launch_t(const AgWsArgs& a, int64_t tiles, hipStream_t stream) {
    const int gx = grid_for(tiles);  // one block per tile, striding beyond the cap
    hipLaunchKernelGGL((ag_ws_kernel<T, KS, NT, ANY>), dim3(gx), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int KS, bool ANY, typename... Args>
hipError_t pick_nt(const Args&... a) {
    return tuning().ag_nontemporal ? launch_t<T, KS, true, ANY>(a...) : launch_t<T, KS, false, ANY>(a...);
}

// K = 8 specialised; full buffers in different phases take the generic
// kernel built for them
template <typename T, typename... Args>
hipError_t pick_k(int K, bool any, const Args&... a) {
    if (any) return pick_nt<T, 0, true>(a...);
    switch (K) {
        case 8: return pick_nt<T, 8, false>(a...);
        default: return pick_nt<T, 0, false>(a...);
    }
}

// The segment records of a launch (empty segments dropped): vector mask and
// tiles per chunk of each, and the running first tile. *any: the full
// buffers sit in different 16-byte phases (the kernels built for that).
int64_t describe(int K, const ConstPtrs& shards, const MutPtrs& fulls, zr_dtype dt, const zr_seg* segs,
                 int n_segs, AgSeg* out, int64_t* unit0, int* used, int* fphase, bool* any) {
    const int es = dt == ZR_BF16 ? 2 : 4;
    const int64_t tile = dt == ZR_BF16 ? kAgTile<uint16_t> : kAgTile<float>;  // elements per tile
    // whole units from registers need one destination grid for all K full
    // buffers (their bases in one phase within 16 bytes); a chunk's source is
    // one shard, so the shards may sit anywhere. Full buffers in different
    // phases stage the source in LDS, and their tiles cover up to
    // 16 / es - 1 elements before a chunk. ZR_FORCE_PATH=element: every chunk
    // element-wise
    const uintptr_t fph = (uintptr_t)fulls.p[0] & 15;
    const bool allowed = tuning().force_path != kPathElement;
    bool same = true;
    for (int r = 0; r < K; ++r) same = same && (((uintptr_t)fulls.p[r]) & 15) == fph;
    const bool bases = allowed && same;
    *any = allowed && !same;
    if (fphase) *fphase = (int)(fph / es);
    int n = 0;
    int64_t units = 0;
    for (int s = 0; s < n_segs; ++s) {
        if (segs[s].numel == 0) continue;
        unit0[n] = units;
        AgSeg& d = out[n++];
        d.shard_off = segs[s].shard_off;
        d.full_off = segs[s].full_off;
        d.numel = segs[s].numel;
        d.C = (d.numel + K - 1) / K;
        d.pad_ = 0;
        // with 16-byte aligned bases every chunk moves whole units, on its
        // destination's grid: its units start up to 16 / es - 1 elements
        // before the chunk (the lead), which its tiles must also cover
        d.vec_mask = 0;
        int64_t lead = *any ? 16 / es - 1 : 0;
        if (bases) {
            for (int j = 0; j < K; ++j) {
                d.vec_mask |= 1ull << j;
                const int64_t l = ((int64_t)(fph / es) + d.full_off + (int64_t)j * d.C) & (16 / es - 1);
                lead = l > lead ? l : lead;
            }
        }
        d.tiles_per_chunk = (int)((d.C + lead + tile - 1) / tile);
        units += (int64_t)K * d.tiles_per_chunk;
    }
    unit0[n] = units;
    *used = n;
    return units;
}

}  // namespace

hipError_t launch_all_gather(int K, const ConstPtrs& shards, const MutPtrs& fulls, zr_dtype dt,
                             const zr_seg* segs, int n_segs, int shift, hipStream_t stream) {
    AgArgs a;
    a.c.shards = shards;
    a.c.fulls = fulls;
    a.c.K = K;
    a.c.shift = shift;
    int used = 0;
    bool any = false;
    if (describe(K, shards, fulls, dt, segs, n_segs, a.seg, a.unit0, &used, &a.c.fphase, &any) == 0)
        return hipSuccess;
    a.nseg = used;
    if (dt == ZR_BF16) return pick_k<uint16_t>(K, any, a, stream);
    return pick_k<float>(K, any, a, stream);
}

hipError_t launch_all_gather_ws(int K, const ConstPtrs& shards, const MutPtrs& fulls, zr_dtype dt,
                                const zr_seg* segs, int n_segs, int shift, void* ws,
                                hipStream_t stream) {
    std::vector<uint8_t> image(ag_table_bytes(n_segs));
    int64_t* unit0 = reinterpret_cast<int64_t*>(image.data());
    AgSeg* recs = reinterpret_cast<AgSeg*>(image.data() + 8 * (size_t)(n_segs + 1));
    int used = 0;
    int fphase = 0;
    bool any = false;
    const int64_t tiles = describe(K, shards, fulls, dt, segs, n_segs, recs, unit0, &used, &fphase, &any);
    if (tiles == 0) return hipSuccess;
    // the records were written compactly after n_segs + 1 first-tile slots; the
    // kernel reads used + 1 of them and used records
    AgWsArgs a;
    a.c.shards = shards;
    a.c.fulls = fulls;
    a.c.K = K;
    a.c.shift = shift;
    a.c.fphase = fphase;
    a.unit0 = (uint64_t)(uintptr_t)ws;
    a.seg = (uint64_t)(uintptr_t)ws + 8 * (uint64_t)(n_segs + 1);
    a.nseg = used;
    const size_t bytes = 8 * (size_t)(n_segs + 1) + sizeof(AgSeg) * (size_t)used;
    hipError_t e = stage_table(ws, image.data(), bytes, stream, true);
    if (e != hipSuccess) return e;
    if (dt == ZR_BF16) return pick_k<uint16_t>(K, any, a, tiles, stream);
    return pick_k<float>(K, any, a, tiles, stream);
}

}  // namespace zr
