// Reduce-scatter straight from fragmented gradients: the discrete path.
//
// ZeRO-3 reduces a bucket either from its contiguous flat buffer or, when the
// gradients stayed fragmented, through a reduce-scatter over the list of
// per-parameter gradients ("DeepSpeed ZeRO-3 源码解析", 5.2, the discrete
// path; 3.2 on when gradients stay fragmented). Here the result is defined as
// flattening the fragments into a virtual bucket of N elements (fragment p at
// offset n_0 + ... + n_{p-1}, zero padding after the last one up to K*C) and
// reducing that bucket exactly as the contiguous reduce-scatter does: chunk
// j = g / C folded in its order, averaged, written to rank (j - shift) mod K
// at g - jC. The bucket itself is never written: each input element is read
// once from its fragment.
//
// Work is cut into segments: the part of one fragment that falls in one
// chunk. A segment is a contiguous run of the fragment on every rank that
// lands contiguously in one holder's partition, so it is reduced like a chunk
// of the contiguous kernel: the same 4-wave x S-slice x 256-element tiles of
// lane-owned quads, every rank's loads in flight before the ring-order adds,
// non-temporal streams. The descriptor table (each fragment's rank pointers,
// offset and size; each segment's fragment, chunk, head and first tile)
// rides in the kernel arguments when it fits one argument block: up to 32
// fragments and 256 rank pointers (the padding entry, which has none, takes a
// spare slot after them) and 96 segments, more going out as further
// launches. Given a workspace, a larger table is staged there instead and one
// launch covers every fragment, however many there are (the pages' point in
// bucketing: one operation per bucket, not one per parameter, section 3.1);
// the kernel then reads it with scalar loads and finds a tile's segment with
// a wave-wide search. The grid has one block per tile of the launch, in
// order, so blocks stay balanced however unequal the fragments are, and the
// blocks in flight work on one compact window of memory (a persistent grid
// striding over the tiles ran 7-15% slower). A segment starts its vector
// tiles at a 128-byte line of rank j whose output lies less than a line
// after a 16 KiB boundary of the partition, as the contiguous kernel does:
// the head before it goes to head tiles of its own (as quads, and its edge
// elements one by one), the last tile folds its whole quads as vectors and
// the last few elements one by one, and a full tile whose partition side is
// off the quad grid realigns its results through LDS. When the segment's
// rank runs sit in different quad phases, the tiles lie on rank j's quads and
// every other rank's quad is read as the two aligned quads holding it,
// joined in registers (element by element, such segments ran 4.7-5x slower
// at K = 16-64 and 13% slower at K = 8). A launch holding such a segment
// runs kernels that read every segment this way, so the kernels of aligned
// launches keep their register budget. Under ZR_FORCE_PATH=element every
// segment folds element by element, 1024 elements per tile. The padding
// entry has null pointers, starts its tiles on a 16 KiB boundary of the
// partition and writes +0 (old + 0 when accumulating).
//
// The kernels live in this header; each (input, output) dtype pair is
// instantiated in a translation unit of its own (zr_rsf_<in>_<out>.hip) so
// the four compile in parallel, and the host planning code in zr_rsf.hip
// picks among them through rsf::pick_avg.
#pragma once

#include <cstdint>

#include "zr_fold_any.hpp"

namespace zr {
namespace rsf {

// Entry slots: kRsfEntriesPerLaunch fragments with rank pointers, plus one
// more for the padding entry, which has none.
constexpr int kRsfSlots = kRsfEntriesPerLaunch + 1;

// Flag in a segment's head: its rank runs sit in different quad phases, and
// its vector tiles read each rank's quads as aligned pairs joined in
// registers (a head is below 16 KiB / 2 + a line of elements, so the flag
// never meets a head's own bits).
constexpr int kAnyPhase = 1 << 14;

// Fields every launch carries, whichever table it reads.
struct RsfCommon {
    MutPtrs out;
    int64_t C;
    int K, shift, accumulate;
    int pad_m;  // the padding entry (writes +0), -1: none
    float inv_k, kf;
};

// A launch whose table rides in its kernel arguments.
struct RsfArgs {
    RsfCommon c;
    const void* ptr[kRsfPtrsPerLaunch];    // entry-major: ptr[m * K + r]
    int64_t off[kRsfSlots];                // virtual-bucket offset of entry m
    int64_t n[kRsfSlots];                  // elements of entry m
    int32_t tile0[kRsfSegsPerLaunch + 1];  // first tile of segment s; tile0[nseg] = all tiles
    uint8_t seg_m[kRsfSegsPerLaunch];      // entry of segment s
    uint8_t seg_j[kRsfSegsPerLaunch];      // chunk of segment s
    int16_t seg_head[kRsfSegsPerLaunch];   // vector tiles start at this offset (| kAnyPhase); -1: element-wise
    int nseg;
};
static_assert(sizeof(RsfArgs) <= 4096, "discrete reduce-scatter arguments exceed 4 KB");

// A launch whose table is staged in a workspace: device addresses of its
// arrays (the layout of rsf_table_bytes).
struct RsfWsArgs {
    RsfCommon c;
    uint64_t tile0;  // int64_t[nseg + 1]: first tile of segment s; tile0[nseg] = all tiles
    uint64_t seg;    // int32_t[3 * nseg]: entry, chunk and head of segment s at 3s
    uint64_t ent;    // int64_t[2 * nent]: virtual-bucket offset and size of entry m at 2m
    uint64_t ptr;    // const void*[K * nent], entry-major (null for the padding entry)
    int64_t nseg;
};

// One segment's record and one entry's record.
struct SegRec {
    int m, j, h;  // entry, chunk, head
};
struct EntRec {
    int64_t off, n;
};

// The two table sources behind one interface.
struct ArgTable {
    using Index = int;  // argument launches keep tile numbers within 32 bits
    const RsfArgs& a;
    __device__ __forceinline__ int64_t total() const { return a.tile0[a.nseg]; }
    // a block's tiles only grow, so its last segment is a lower bound
    __device__ __forceinline__ int64_t find(int64_t from, int64_t t) const {
        return find_slot(a.tile0, a.nseg, (int)from, (int)t);
    }
    __device__ __forceinline__ int64_t first(int64_t s) const { return a.tile0[s]; }
    __device__ __forceinline__ SegRec seg(int64_t s) const { return {a.seg_m[s], a.seg_j[s], a.seg_head[s]}; }
    __device__ __forceinline__ EntRec ent(int m) const { return {a.off[m], a.n[m]}; }
    __device__ __forceinline__ const void* ptr(int m, int K, int r) const { return a.ptr[m * K + r]; }
};

struct WsTable {
    using Index = int64_t;
    cptr<int64_t> tile0;
    cptr<int32_t> sg;
    cptr<int64_t> en;
    cptr<const void*> ptrs;
    int64_t nseg;
    __device__ __forceinline__ explicit WsTable(const RsfWsArgs& a)
        : tile0(table_at<int64_t>(a.tile0)), sg(table_at<int32_t>(a.seg)), en(table_at<int64_t>(a.ent)),
          ptrs(table_at<const void*>(a.ptr)), nseg(a.nseg) {}
    __device__ __forceinline__ int64_t total() const { return tile0[nseg]; }
    __device__ __forceinline__ int64_t find(int64_t, int64_t t) const { return find_slot64(tile0, nseg, t); }
    __device__ __forceinline__ int64_t first(int64_t s) const { return tile0[s]; }
    __device__ __forceinline__ SegRec seg(int64_t s) const { return {sg[3 * s], sg[3 * s + 1], sg[3 * s + 2]}; }
    __device__ __forceinline__ EntRec ent(int m) const { return {en[2 * (int64_t)m], en[2 * (int64_t)m + 1]}; }
    __device__ __forceinline__ const void* ptr(int m, int K, int r) const { return ptrs[(int64_t)m * K + r]; }
};

// Elements per tile of a segment that folds element by element (4 per thread).
constexpr int64_t kElemTile = kThreads * 4;

template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S, bool ANY, typename Tab>
__device__ __forceinline__ void rsf_body(const RsfCommon& c, const Tab& tab) {
    constexpr int64_t T = kRsTileOf<S>;
    constexpr bool kStatic = ORDER != kFree && KS > 0 && KS <= 8;
    const int K = KS > 0 ? KS : c.K;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // per wave, one full tile's results in span order (tiles whose partition
    // side is off the quad grid)
    __shared__ float stage[kThreads / 64][S * 256];
    using Index = typename Tab::Index;
    const Index total = (Index)tab.total();
    Index s = 0;
    for (Index t = blockIdx.x; t < total; t += gridDim.x) {
        s = (Index)tab.find(s, t);
        const SegRec sr = tab.seg(s);
        const int m = sr.m, j = sr.j;
        const EntRec er = tab.ent(m);
        const int64_t jc = (int64_t)j * c.C;
        const int64_t f0 = er.off, f1 = er.off + er.n;
        const int64_t lo = f0 > jc ? f0 : jc;
        const int64_t hi = f1 < jc + c.C ? f1 : jc + c.C;
        const int64_t l_lo = lo - f0, len = hi - lo;  // fragment-local start, length
        TOut* outp = static_cast<TOut*>(c.out.p[wrap(j - c.shift + K, K)]) + (lo - jc);
        auto ptr = [=](int r) __attribute__((always_inline)) { return tab.ptr(m, K, r); };
        const bool pad = m == c.pad_m;
        const int64_t tt = t - tab.first(s);
        // the head without the flag of segments whose ranks sit in
        // different quad phases (only the kernels built for them see it)
        const int64_t h = (ANY && sr.h >= 0) ? (sr.h & (kAnyPhase - 1)) : sr.h;

        // one output element (segment offset o), folded element-wise
        auto elem = [&](int64_t o) __attribute__((always_inline)) {
            float v = 0.0f;
            if (!pad) v = average<AVG>(fold_elem<TIn, KS, ORDER>(ptr, K, j, l_lo + o), c.inv_k, c.kf);
            if (c.accumulate) v = __fadd_rn(load_elem(outp + o), v);
            store_elem(outp + o, v);
        };
        if (h < 0) {
            const int64_t e0 = tt * kElemTile, e1 = (e0 + kElemTile < len) ? e0 + kElemTile : len;
            for (int64_t o = e0 + threadIdx.x; o < e1; o += kThreads) elem(o);
            continue;
        }
        // the partition side is quad aligned at the vector tiles' start or not
        // at all (the tiles advance in whole quads)
        const bool out_quad = (((uintptr_t)(outp + h)) & (4 * sizeof(TOut) - 1)) == 0;
        // one result v for segment offset o: accumulate, store
        auto put1 = [&](int64_t o, float v) __attribute__((always_inline)) {
            if (c.accumulate) v = __fadd_rn(load_elem(outp + o), v);
            store_elem(outp + o, v);
        };
        // A full tile's S folded quads at segment offsets o0 + 256k when the
        // partition side is d = 1-3 elements past a quad boundary. A wave's S
        // slices cover one contiguous span of S * 256 results: the wave puts
        // them in its LDS stage in order, every lane reads back the aligned
        // quad that starts 4 - d results into its own (the next lane's first
        // results complete it) and stores it with one aligned store; the 4 - d
        // results before the span's first boundary and the d after its last are
        // then stored one by one by lanes 0 and 63. (Storing every result
        // singly made these tiles store-bound: 4x the store instructions.)
        auto emit_staged = [&](int64_t o0, float (&acc)[S][4]) __attribute__((always_inline)) {
            if (!pad) {
#pragma unroll
                for (int k = 0; k < S; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[k][e] = average<AVG>(acc[k][e], c.inv_k, c.kf);
            }
            float* st = stage[wave];
            __syncthreads();  // the stage's previous contents have been read
#pragma unroll
            for (int k = 0; k < S; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[256 * k + 4 * lane + e] = acc[k][e];
            __syncthreads();
            const int d = (int)((((uintptr_t)(outp + h)) / sizeof(TOut)) & 3);  // uniform, 1..3
            const int sh = 4 - d;
            const int64_t ow = o0 - 4 * lane;  // the span's first result
#pragma unroll
            for (int k = 0; k < S; ++k) {
                const int p = 256 * k + 4 * lane + sh;  // span index of this lane's aligned quad
                if (p + 4 > S * 256) continue;           // lane 63 of the last slice: the tail
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = st[p + e];
                TOut* dst = outp + ow + p;  // quad aligned
                if (c.accumulate) {
                    float old[4];
                    widen4(load_quad<TOut, NT>(dst), old);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __fadd_rn(old[e], v[e]);
                }
                store_quad<TOut, NT>(dst, pack4<TOut>(v));
            }
            if (lane == 0) {
#pragma unroll
                for (int e = 0; e < 3; ++e)
                    if (e < sh) put1(ow + e, st[e]);
            }
            if (lane == 63) {
#pragma unroll
                for (int e = 1; e < 4; ++e)
                    if (e >= sh) put1(ow + S * 256 - 4 + e, st[S * 256 - 4 + e]);
            }
        };
        // SS folded quads at segment offsets o0 + 256k: average, accumulate, store
        auto emit = [&](int64_t o0, auto& acc, auto slices) __attribute__((always_inline)) {
            constexpr int SS = decltype(slices)::value;
            if (!pad) {
#pragma unroll
                for (int k = 0; k < SS; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[k][e] = average<AVG>(acc[k][e], c.inv_k, c.kf);
            }
            if (out_quad) {
                if (c.accumulate) {
#pragma unroll
                    for (int k = 0; k < SS; ++k) {
                        float old[4];
                        widen4(load_quad<TOut, NT>(outp + o0 + 256 * k), old);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[k][e] = __fadd_rn(old[e], acc[k][e]);
                    }
                }
#pragma unroll
                for (int k = 0; k < SS; ++k) store_quad<TOut, NT>(outp + o0 + 256 * k, pack4<TOut>(acc[k]));
            } else {
#pragma unroll
                for (int k = 0; k < SS; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        TOut* o = outp + o0 + 256 * k + e;
                        float v = acc[k][e];
                        if (c.accumulate) v = __fadd_rn(load_elem(o), v);
                        store_elem(o, v);
                    }
            }
        };
        // SS quads of the fragment (zeros for the padding entry)
        auto fold = [&](int64_t o0, auto& acc, auto slices) __attribute__((always_inline)) {
            constexpr int SS = decltype(slices)::value;
            if (pad) {
#pragma unroll
                for (int k = 0; k < SS; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[k][e] = 0.0f;
            } else if constexpr (ANY) {
                // every segment of such a launch, since a rank in the tiles'
                // phase costs only a repeated load (one fold per call site
                // keeps these kernels small); the tiles' quads sit at segment
                // offsets congruent to h mod 4
                if constexpr (ORDER == kFree)
                    fold_free_quads_any<TIn, KS, NT, SS>(ptr, K, l_lo + o0, l_lo + h, acc);
                else
                    fold_ring_quads_any<TIn, KS, NT, SS, ORDER == kWire>(ptr, K, j, l_lo + o0, l_lo + h, acc);
            } else {
                const RingBases<TIn, kStatic ? KS : 1> bases(ptr, kStatic ? j : 0);
                fold_quads<TIn, KS, NT, SS, ORDER, kStatic>(bases, ptr, K, j, l_lo + o0, acc);
            }
        };
        // head tiles over [0, min(h, len)), ceil(that / T) of them, then tiles
        // over [h, len), the last one possibly partial. Head tile tt covers
        // [tt T, min((tt+1) T, hc)): quads on the tiles' quad grid (offsets
        // congruent to h mod 4), its other elements one by one
        const int64_t hc = h < len ? h : len;
        const int64_t nh = (hc + T - 1) / T;
        if (tt < nh) {
            const int64_t lo = tt * T;
            const int64_t hi = lo + T < hc ? lo + T : hc;
            const int64_t q0 = lo + (h & 3);  // lo is a multiple of 4
            for (int64_t o = lo + threadIdx.x; o < q0 && o < hi; o += kThreads) elem(o);
            const int64_t qe = hi > q0 ? q0 + ((hi - q0) & ~(int64_t)3) : q0;
#pragma unroll 1
            for (int64_t q = q0 + (int64_t)threadIdx.x * 4; q < qe; q += kThreads * 4) {
                float acc[1][4];
                fold(q, acc, std::integral_constant<int, 1>{});
                emit(q, acc, std::integral_constant<int, 1>{});
            }
            for (int64_t o = (qe > lo ? qe : lo) + threadIdx.x; o < hi; o += kThreads) elem(o);
            continue;
        }
        const int64_t ot = h + (tt - nh) * T;
        if (ot >= len) continue;
        const int64_t o0 = ot + (int64_t)wave * (S * 256) + lane * 4;
        if (ot + T <= len) {
            float acc[S][4];
            fold(o0, acc, std::integral_constant<int, S>{});
            if (out_quad)
                emit(o0, acc, std::integral_constant<int, S>{});
            else
                emit_staged(o0, acc);
        } else {
#pragma unroll 1
            for (int k = 0; k < S; ++k) {
                const int64_t q = o0 + 256 * k;
                if (q + 4 <= len) {
                    float acc[1][4];
                    fold(q, acc, std::integral_constant<int, 1>{});
                    emit(q, acc, std::integral_constant<int, 1>{});
                } else {
#pragma unroll 1
                    for (int e = 0; e < 4; ++e)
                        if (q + e < len) elem(q + e);
                }
            }
        }
    }
}

template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S, bool ANY>
__global__ void __launch_bounds__(kThreads) rsf_kernel(const RsfArgs a) {
    rsf_body<TIn, TOut, KS, AVG, ORDER, NT, S, ANY>(a.c, ArgTable{a});
}

template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S, bool ANY>
__global__ void __launch_bounds__(kThreads) rsf_ws_kernel(const RsfWsArgs a) {
    rsf_body<TIn, TOut, KS, AVG, ORDER, NT, S, ANY>(a.c, WsTable(a));
}

using LaunchFn = hipError_t (*)(const RsfArgs&, hipStream_t);
using WsLaunchFn = hipError_t (*)(const RsfWsArgs&, int64_t, hipStream_t);

template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S, bool ANY>
hipError_t launch_t(const RsfArgs& a, hipStream_t stream) {
    const int gx = grid_for(a.tile0[a.nseg]);  // one block per tile
    hipLaunchKernelGGL((rsf_kernel<TIn, TOut, KS, AVG, ORDER, NT, S, ANY>), dim3(gx), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S, bool ANY>
hipError_t launch_ws_t(const RsfWsArgs& a, int64_t tiles, hipStream_t stream) {
    const int gx = grid_for(tiles);  // one block per tile, striding beyond the cap
    hipLaunchKernelGGL((rsf_ws_kernel<TIn, TOut, KS, AVG, ORDER, NT, S, ANY>), dim3(gx), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

struct Fns {
    LaunchFn args;
    WsLaunchFn ws;
};
template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S, bool ANY = false>
constexpr Fns fns() {
    return {&launch_t<TIn, TOut, KS, AVG, ORDER, NT, S, ANY>, &launch_ws_t<TIn, TOut, KS, AVG, ORDER, NT, S, ANY>};
}

// Ring and wire order at K = 8 specialised, the rest generic (batches of
// eight ranks in flight, four in the wire order; the free and generic wire
// kernels keep at most four slices per wave); fp32 input makes the wire
// order the ring order. Small plans in the ring order use one slice per wave. Plans with segments
// whose ranks sit in different quad phases take the generic kernels built to
// read them.
template <typename TIn, typename TOut, int AVG>
Fns pick_k(int K, int order, bool small, bool any) {
    constexpr int S = kSlices<TIn, TOut>;
    constexpr int SG = kSlicesGeneric<TIn, TOut>;  // the tiles rs_generic_narrow() plans
    constexpr bool NT = kRsNontemporal;
    if (any) {  // at most four slices per wave in every order (the planner's tiles)
        if (order == kFree) return fns<TIn, TOut, 0, AVG, kFree, NT, SG, true>();
        if (order == kWire && sizeof(TIn) == 2) return fns<TIn, TOut, 0, AVG, kWire, NT, SG, true>();
        return small ? fns<TIn, TOut, 0, AVG, kRing, NT, 1, true>() : fns<TIn, TOut, 0, AVG, kRing, NT, SG, true>();
    }
    if (order == kFree) return fns<TIn, TOut, 0, AVG, kFree, NT, SG>();
    if (order == kWire && sizeof(TIn) == 2) {
        if (K == 8) return fns<TIn, TOut, 8, AVG, kWire, NT, S>();
        return fns<TIn, TOut, 0, AVG, kWire, NT, SG>();
    }
    if (K == 8) return small ? fns<TIn, TOut, 8, AVG, kRing, NT, 1>() : fns<TIn, TOut, 8, AVG, kRing, NT, S>();
    return small ? fns<TIn, TOut, 0, AVG, kRing, NT, 1>() : fns<TIn, TOut, 0, AVG, kRing, NT, S>();
}

template <typename TIn, typename TOut>
Fns pick_avg(int K, int avg, int order, bool small, bool any) {
    switch (avg) {
        case 1: return pick_k<TIn, TOut, 1>(K, order, small, any);
        case 2: return pick_k<TIn, TOut, 2>(K, order, small, any);
        default: return pick_k<TIn, TOut, 0>(K, order, small, any);
    }
}

// The four dtype pairs are instantiated in their own translation units.
extern template Fns pick_avg<uint16_t, float>(int, int, int, bool, bool);
extern template Fns pick_avg<uint16_t, uint16_t>(int, int, int, bool, bool);
extern template Fns pick_avg<float, float>(int, int, int, bool, bool);
extern template Fns pick_avg<float, uint16_t>(int, int, int, bool, bool);

}  // namespace rsf
}  // namespace zr
