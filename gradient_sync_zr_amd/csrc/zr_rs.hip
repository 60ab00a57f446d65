// Fused reduce-scatter + average + cast.
//
// For holder rank q and chunk-local offset o, with j = (q + shift) mod K and
// g = j*C + o, the kernel folds in_{j}[g], in_{j+1}[g], ..., in_{j-1}[g] in
// ring order in fp32 ("图解 Ring All-Reduce", Phase 1: chunk j starts at rank
// j, gains one addend per hop and ends on rank j-1 after K-1 hops, which is
// shift = 1; the ZeRO-3 contiguous path keeps slice r on rank r, shift = 0,
// "DeepSpeed ZeRO-3 源码解析" 5.2), divides by K (CMU 11-868 lecture 14 notes,
// 4.1: SUM then divide by the world size), and writes the holder's partition
// once, in fp32 or rounded once to bf16 (the single bf16 -> fp32 cast of the
// ZeRO-3 data flow, section 1, moved into the reduction's only write).
//
// Grid: one block per tile, tiles numbered by pairs of chunks (chunks 0
// and 1, then 2 and 3, ...), consecutive blocks alternating between the
// pair's two chunks, so the blocks the dispatcher has in flight work on two
// compact windows of the address space; a block finds its chunk j, and with
// it the holder and every rank pointer, uniformly from the pairs' first
// tiles. (Two chunks at a time ran 1-2% faster than one; four or eight ran
// 2-4% slower. A persistent grid striding over the tiles ran 7-8% slower:
// its blocks drift apart over the chunk.) A tile is 4 waves x S
// slices x 256 elements; lane l of a wave owns elements 4l..4l+3 of each of
// its slices, so each load instruction reads, and each store instruction
// writes, one contiguous span of whole cache lines. All K ranks' loads of
// all S slices are issued before the first add. Loads and stores are
// non-temporal by default: every byte is touched exactly once.
//
// In a chunk whose start j*C allows quad access (j*C a multiple of 4), the
// vector tiles begin at an input element that starts a 128-byte line, so
// the K input streams are read in whole lines, and whose output lies less
// than a line after a 16 KiB boundary of the holder's partition, so the
// tiles' writes fill aligned 16 KiB blocks. The head before that point (at
// most 16 KiB of output plus a line) is cut into head tiles of its own, so
// no block does more than a tile's work (one block folding the whole head
// set the time of small launches): whole quads as vectors, its last few
// elements one by one. The last tile folds its whole quads below N as
// vectors and the few elements after them one by one. A call in which some
// chunk's start does not allow quad access (or whose bases are not quad
// aligned) never reaches this kernel: it goes out as the discrete
// reduce-scatter over one fragment per rank (via_fragments, below).
// Positions g >= N are padding and receive +0.
#include <algorithm>
#include <new>

#include "zr_fold.hpp"

namespace zr {
namespace {

// Output block the vector tiles' writes are aligned to (bytes).
constexpr uintptr_t kOutBlock = 16384;

struct RsArgs {
    ConstPtrs in;
    MutPtrs out;
    int64_t N, C;
    uint64_t vec_mask;         // bit j: chunk j allows the vector path (all set, or the host routes the call)
    int16_t head[kMaxRanks];   // chunk j's vector tiles start at chunk offset head[j]
    int64_t tile0[kMaxRanks + 1];      // first tile of chunk group q; tile0[ngroups] = all tiles
    int64_t ntile[kMaxRanks];          // tiles of chunk j
    int ngroups;                       // ceil(K / group)
    int group;                         // chunks per group: 1, or 2 (a pair's blocks alternate)
    int K, shift;
    int accumulate;            // 1: out = old + result (gradient accumulation)
    float inv_k, kf;
};
static_assert(sizeof(RsArgs) <= 4096, "reduce-scatter arguments exceed 4 KB");

template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S>
__global__ void __launch_bounds__(kThreads) rs_kernel(const RsArgs a) {
    constexpr int64_t T = kRsTileOf<S>;
    constexpr bool kStatic = ORDER != kFree && KS > 0 && KS <= 8;
    const int K = KS > 0 ? KS : a.K;
    const int64_t C = a.C, N = a.N;
    auto ptr = [&](int r) __attribute__((always_inline)) { return a.in.p[r]; };
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    // one tile per block; a launch capped below the tile count strides
    for (int64_t i = blockIdx.x; i < a.tile0[a.ngroups]; i += gridDim.x) {
        // the tile's chunk group: the last q with tile0[q] <= i (uniform);
        // the two chunks of a pair take alternate blocks
        int q = 0;
        for (int hi = a.ngroups; hi - q > 1;) {
            const int mid = (q + hi) >> 1;
            if (a.tile0[mid] <= i)
                q = mid;
            else
                hi = mid;
        }
        const int64_t w = i - a.tile0[q];
        const int first = a.group * q;
        const bool two = a.group == 2 && first + 1 < K;
        const int j = two ? first + (int)(w & 1) : first;
        const int64_t t = two ? (w >> 1) : w;
        if (t >= a.ntile[j]) continue;  // the pair's shorter chunk has run out
        const int holder = wrap(j - a.shift + K, K);
        const int64_t chunk_base = (int64_t)j * C;
        TOut* outp = static_cast<TOut*>(a.out.p[holder]);
        const RingBases<TIn, kStatic ? KS : 1> bases(ptr, kStatic ? j : 0);

        // one output element, folded element-wise (padding past N gets +0)
        auto elem = [&](int64_t o) __attribute__((always_inline)) {
            const int64_t g = chunk_base + o;
            float s = 0.0f;
            if (g < N) {
                s = fold_elem<TIn, KS, ORDER>(ptr, K, j, g);
                s = average<AVG>(s, a.inv_k, a.kf);
            }
            if (a.accumulate) s = __fadd_rn(load_elem(outp + o), s);
            store_elem(outp + o, s);
        };
        // SS folded quads at chunk offsets o0 + 256k: average, accumulate, store
        auto emit = [&](int64_t o0, auto& acc, auto slices) __attribute__((always_inline)) {
            constexpr int SS = decltype(slices)::value;
#pragma unroll
            for (int k = 0; k < SS; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[k][e] = average<AVG>(acc[k][e], a.inv_k, a.kf);
            if (a.accumulate) {
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
        };

        // the chunk's tiles: first ceil(min(h, C) / T) head tiles over
        // [0, h), then tiles over [h, C), the last one possibly partial
        const int64_t h = a.head[j];
        const int64_t valid = (N - chunk_base < C) ? N - chunk_base : C;  // non-padding extent
        const int64_t hc = h < C ? h : C;
        const int64_t nh = (hc + T - 1) / T;
        if (t < nh) {
            // head tile t covers [tT, min((t+1)T, hc)) on the tiles' quad grid
            // (the chunk start is a quad boundary): a whole tile of whole quads
            // below the padding folds as a main tile does; otherwise its whole
            // quads below the padding fold as vectors (one slice per pass) and
            // its other elements one by one
            const int64_t lo = t * T;
            const int64_t hi = lo + T < hc ? lo + T : hc;
            if (hi - lo == T && hi <= valid) {
                const int64_t o0 = lo + (int64_t)wave * (S * 256) + lane * 4;
                float acc[S][4];
                fold_quads<TIn, KS, NT, S, ORDER, kStatic>(bases, ptr, K, j, chunk_base + o0, acc);
                emit(o0, acc, std::integral_constant<int, S>{});
                continue;
            }
            const int64_t lim = (valid < hi ? valid : hi) & ~(int64_t)3;  // < lo: no whole quad
#pragma unroll 1
            for (int64_t o4 = lo + (int64_t)threadIdx.x * 4; o4 + 4 <= lim; o4 += kThreads * 4) {
                float acc[1][4];
                fold_quads<TIn, KS, NT, 1, ORDER, kStatic>(bases, ptr, K, j, chunk_base + o4, acc);
                emit(o4, acc, std::integral_constant<int, 1>{});
            }
            for (int64_t o = (lim > lo ? lim : lo) + threadIdx.x; o < hi; o += kThreads) elem(o);
            continue;
        }
        const int64_t ot = h + (t - nh) * T;
        if (ot >= C) continue;
        const int64_t o0 = ot + (int64_t)wave * (S * 256) + lane * 4;
        if (ot + T <= valid) {
            float acc[S][4];
            fold_quads<TIn, KS, NT, S, ORDER, kStatic>(bases, ptr, K, j, chunk_base + o0, acc);
            emit(o0, acc, std::integral_constant<int, S>{});
        } else {
            // the last tile: whole quads below the padding fold as vectors,
            // the rest up to C element by element
#pragma unroll 1
            for (int k = 0; k < S; ++k) {
                const int64_t q = o0 + 256 * k;
                if (q + 4 <= valid) {
                    float acc[1][4];
                    fold_quads<TIn, KS, NT, 1, ORDER, kStatic>(bases, ptr, K, j, chunk_base + q, acc);
                    emit(q, acc, std::integral_constant<int, 1>{});
                } else {
#pragma unroll 1
                    for (int e = 0; e < 4; ++e)
                        if (q + e < C) elem(q + e);
                }
            }
        }
    }
}

// One block per tile, up to tuning().max_grid blocks (beyond that they stride).
template <typename TIn, typename TOut, int KS, int AVG, int ORDER, bool NT, int S>
hipError_t launch_t(const RsArgs& a, hipStream_t stream) {
    const int64_t total = a.tile0[a.ngroups];
    const int gx = grid_for(total);
    hipLaunchKernelGGL((rs_kernel<TIn, TOut, KS, AVG, ORDER, NT, S>), dim3(gx), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

// Orders: the free order has one generic instantiation; ring and wire orders
// have K = 8 specialised, other K take the generic kernel (batches of eight
// ranks in flight, four in the wire order). The free and generic wire
// kernels keep at most four slices per wave (kSlicesGeneric). With fp32
// input the wire order is the ring order (rounding every hop to fp32 is what
// the fp32 adds already do). Small launches in the ring order use one slice
// per wave.
using LaunchFn = hipError_t (*)(const RsArgs&, hipStream_t);

template <typename TIn, typename TOut, int AVG>
LaunchFn pick_k(int K, int order, bool small) {
    constexpr int S = kSlices<TIn, TOut>;
    constexpr int SG = kSlicesGeneric<TIn, TOut>;  // the tiles rs_generic_narrow() launches
    constexpr bool NT = kRsNontemporal;
    if (order == kFree) return &launch_t<TIn, TOut, 0, AVG, kFree, NT, SG>;
    if (order == kWire && sizeof(TIn) == 2) {
        if (K == 8) return small ? &launch_t<TIn, TOut, 8, AVG, kWire, NT, 1> : &launch_t<TIn, TOut, 8, AVG, kWire, NT, S>;
        return &launch_t<TIn, TOut, 0, AVG, kWire, NT, SG>;
    }
    if (K == 8) return small ? &launch_t<TIn, TOut, 8, AVG, kRing, NT, 1> : &launch_t<TIn, TOut, 8, AVG, kRing, NT, S>;
    return small ? &launch_t<TIn, TOut, 0, AVG, kRing, NT, 1> : &launch_t<TIn, TOut, 0, AVG, kRing, NT, S>;
}

template <typename TIn, typename TOut>
LaunchFn pick_avg(int K, int avg_mode, int order, bool small) {
    switch (avg_mode) {
        case 1: return pick_k<TIn, TOut, 1>(K, order, small);
        case 2: return pick_k<TIn, TOut, 2>(K, order, small);
        default: return pick_k<TIn, TOut, 0>(K, order, small);
    }
}

// Fills the launch geometry of `a` (vector chunks, heads, tiles per chunk and
// pair) and returns the kernel that runs it.
// Reduce-scatters with bf16 input that overwrite their partitions take
// one-slice tiles (1024 elements, 4 KiB of fp32 output) at any size where
// that streamed faster on 500M-element buckets:
//  - K = 8, in the ring order or its bf16-wire variant (the static K = 8
//    kernels, 42-50 VGPRs, eight waves per SIMD): 2-6% faster than 16 KiB
//    tiles, for fp32 and bf16 output (two slices per wave ran slower than
//    either);
//  - K > 8 with fp32 output, in the ring order (the generic kernel, 32
//    ranks' loads in flight per batch): 2-3% faster at K = 16, 32 and 64.
//    With bf16 output K = 16 ran 2% slower, and below K = 8 one-slice tiles
//    carry too little per block (2.1-2.8 TB/s at K = 2-4 against 5.1-5.5).
// With fp32 input, or reading the partition back, the four-slice tiles stayed
// 2-7% ahead, and so did they for the discrete reduce-scatter of one layer's
// gradients (6%).
template <typename TIn, typename TOut>
constexpr bool ring_one_slice(int K, int order, bool accumulate) {
    if (sizeof(TIn) != 2 || accumulate) return false;
    if (K == 8) return order == kRing || order == kWire;
    return order == kRing && sizeof(TOut) == 4 && K > 8;
}

template <typename TIn, typename TOut>
LaunchFn prepare_typed(RsArgs& a, int avg_mode, int order) {
    constexpr int64_t T = kRsTile<TIn, TOut>;
    const int fp = tuning().force_path;
    // fewer than two full tiles per CU for each eight ranks (a tile's bytes
    // grow with K), or a shape that streams faster so at any size
    // (ring_one_slice): one-slice tiles, four times as many
    const int64_t k8 = (a.K + 7) / 8;
    // (the ring order, and the wire order's static K = 8 kernels)
    const bool one_ok = order == kRing || (order == kWire && a.K == 8 && sizeof(TIn) == 2);
    const bool small = one_ok &&
                       (fp == kPathSmall ||
                        (fp != kPathLarge && (ring_one_slice<TIn, TOut>(a.K, order, a.accumulate != 0) ||
                                              ((a.C + T - 1) / T) * a.K < 2LL * k8 * device_cu_count())));
    const int64_t Tl = small ? kRsTileOf<1>
                             : (rs_generic_narrow<TIn>(a.K, order) ? kRsTileOf<kSlicesGeneric<TIn, TOut>> : T);
    // Vector path: every base aligned for quad access (8 bytes for bf16
    // quads, 16 for fp32 quads) and j*C a multiple of 4 elements, so that a
    // vector tile start j*C + head is a quad boundary on the input side and
    // head a quad boundary on the output side. head moves the tile start to
    // a 128-byte line of the input (lines hold 128 / sizeof(TIn) elements, a
    // multiple of 4): the first one at or after the next kOutBlock boundary
    // of the holder's partition, so the tiles' writes fill aligned 16 KiB
    // blocks up to less than a line. (Tiles whose writes straddle those
    // blocks streamed 2-4% slower, worst at half a block off.)
    const uintptr_t in_al = sizeof(TIn) * 4, out_al = sizeof(TOut) * 4;
    const int64_t line = 128 / (int64_t)sizeof(TIn);
    bool bases = fp != kPathElement;
    for (int r = 0; r < a.K; ++r) {
        bases = bases && ((uintptr_t)a.in.p[r] % in_al) == 0;
        bases = bases && ((uintptr_t)a.out.p[r] % out_al) == 0;
    }
    a.vec_mask = 0;
    for (int j = 0; j < kMaxRanks; ++j) a.head[j] = 0;
    for (int j = 0; j < a.K; ++j) {
        const int64_t start = a.C * j;
        if (!bases || (start % 4) != 0) continue;
        a.vec_mask |= 1ull << j;
        const int64_t to_line = (line - start % line) % line;
        const uintptr_t ob = (uintptr_t)a.out.p[((j - a.shift) % a.K + a.K) % a.K];  // holder
        const int64_t to_block = (int64_t)((kOutBlock - ob % kOutBlock) % kOutBlock / sizeof(TOut));
        a.head[j] = (int16_t)(to_block + ((to_line - to_block) % line + line) % line);
    }
    // tiles of each chunk: head tiles over [0, min(head, C)), the others over
    // [head, C); chunks go in pairs, a pair's blocks alternating between its
    // two chunks
    for (int j = 0; j < a.K; ++j) {
        const int64_t h = a.head[j];
        const int64_t hc = h < a.C ? h : a.C;
        a.ntile[j] = (hc + Tl - 1) / Tl + (a.C > h ? (a.C - h + Tl - 1) / Tl : 0);
    }
    a.group = tuning().rs_pairs ? 2 : 1;
    a.ngroups = (a.K + a.group - 1) / a.group;
    int64_t tiles = 0;
    for (int q = 0; q < a.ngroups; ++q) {
        a.tile0[q] = tiles;
        const int first = a.group * q;
        tiles += a.group == 2 && first + 1 < a.K ? 2 * std::max(a.ntile[first], a.ntile[first + 1])
                                                  : a.ntile[first];
    }
    a.tile0[a.ngroups] = tiles;
    return pick_avg<TIn, TOut>(a.K, avg_mode, order, small);
}

}  // namespace

namespace {

// The launch of one reduce-scatter: its arguments and the kernel that runs them.
LaunchFn prepare(RsArgs& a, int K, const ConstPtrs& in, zr_dtype in_dt, int64_t N, const MutPtrs& out,
                 zr_dtype out_dt, int shift, int flags, zr_order order) {
    a.in = in;
    a.out = out;
    a.N = N;
    a.K = K;
    a.C = (N + K - 1) / K;
    a.shift = shift;
    a.inv_k = 1.0f / (float)K;
    a.kf = (float)K;
    a.accumulate = (flags & ZR_ACCUMULATE) ? 1 : 0;
    const bool pow2 = (K & (K - 1)) == 0;
    const int avg_mode = !(flags & ZR_AVERAGE) ? 0 : (pow2 ? 1 : 2);
    const int ord = order == ZR_ORDER_FREE ? kFree : (order == ZR_ORDER_RING_WIRE ? kWire : kRing);
    if (in_dt == ZR_BF16 && out_dt == ZR_FP32) return prepare_typed<uint16_t, float>(a, avg_mode, ord);
    if (in_dt == ZR_BF16 && out_dt == ZR_BF16) return prepare_typed<uint16_t, uint16_t>(a, avg_mode, ord);
    if (in_dt == ZR_FP32 && out_dt == ZR_FP32) return prepare_typed<float, float>(a, avg_mode, ord);
    return prepare_typed<float, uint16_t>(a, avg_mode, ord);
}

// Chunks whose start j*C is not a quad boundary (or whose bases are not quad
// aligned) would fold element by element here, a memory round trip per eight
// ranks for every element a lane handles: 0.8-1.1 TB/s at K = 32 and 64, and
// at small K, where a round trip carries little data, 0.7-3.3 TB/s at K = 2-5.
// The discrete reduce-scatter over the same data reads quads on the input's
// own grid and stores single elements only where the partition side is not
// quad aligned (4.3-6.0 TB/s on the same shapes; at K = 8 and 1 GB, 10-46%
// faster). Such a call therefore goes out as that discrete reduce-scatter over
// one fragment per rank (the whole buffer) and the zero padding up to K*C:
// the bucket it describes is the input itself, so every ring-order result is
// the same.
bool via_fragments(const RsArgs& a) {
    const uint64_t all = a.K >= 64 ? ~0ull : ((1ull << a.K) - 1);
    return (a.vec_mask & all) != all;
}

RsfPlan* fragment_plan(int K, const ConstPtrs& in, zr_dtype in_dt, int64_t N, const MutPtrs& out,
                       zr_dtype out_dt, int shift, int flags, zr_order order) {
    const int64_t C = (N + K - 1) / K;
    FragEntry e[2] = {};
    for (int r = 0; r < K; ++r) e[0].ptr[r] = in.p[r];
    e[0].off = 0;
    e[0].n = N;
    int n = 1;
    if ((int64_t)K * C > N) {  // the padding: no pointers
        e[1].off = N;
        e[1].n = (int64_t)K * C - N;
        n = 2;
    }
    return rsf_plan_build(K, e, n, N, in_dt, out, out_dt, shift, flags, order, nullptr);
}

}  // namespace

struct RsPlan {
    RsArgs a;
    LaunchFn fn;
    RsfPlan* frag = nullptr;  // set: the call goes out as this discrete reduce-scatter
};

RsPlan* rs_plan_build(int K, const ConstPtrs& in, zr_dtype in_dt, int64_t N, const MutPtrs& out,
                      zr_dtype out_dt, int shift, int flags, zr_order order) {
    RsPlan* p = new (std::nothrow) RsPlan();
    if (!p) return nullptr;
    p->fn = prepare(p->a, K, in, in_dt, N, out, out_dt, shift, flags, order);
    if (via_fragments(p->a)) {
        p->frag = fragment_plan(K, in, in_dt, N, out, out_dt, shift, flags, order);
        if (!p->frag) {
            delete p;
            return nullptr;
        }
    }
    return p;
}

hipError_t rs_plan_launch(const RsPlan* p, hipStream_t stream) {
    if (p->frag) return rsf_plan_launch(p->frag, stream);
    return p->fn(p->a, stream);
}

void rs_plan_free(RsPlan* p) {
    if (p && p->frag) rsf_plan_free(p->frag);
    delete p;
}

hipError_t launch_reduce_scatter(int K, const ConstPtrs& in, zr_dtype in_dt, int64_t N,
                                 const MutPtrs& out, zr_dtype out_dt, int shift, int flags,
                                 zr_order order, hipStream_t stream) {
    RsArgs a;
    const LaunchFn fn = prepare(a, K, in, in_dt, N, out, out_dt, shift, flags, order);
    if (!via_fragments(a)) return fn(a, stream);
    RsfPlan* f = fragment_plan(K, in, in_dt, N, out, out_dt, shift, flags, order);
    if (!f) return hipErrorOutOfMemory;
    const hipError_t e = rsf_plan_launch(f, stream);
    rsf_plan_free(f);
    return e;
}

}  // namespace zr
