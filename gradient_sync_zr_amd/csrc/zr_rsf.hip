// Reduce-scatter straight from fragmented gradients: the discrete path.
//
// ZeRO-3 reduces a bucket either from its contiguous flat buffer or, when the
// gradients stayed fragmented, through a reduce-scatter over the list of
// per-parameter gradients ("DeepSpeed ZeRO-3 源码解析", 5.2, the discrete
// path; 3.2 on when gradients stay fragmented). Here the result is defined as
// flattening the fragments into a virtual bucket of N elements (fragment p at
// offset n_0 + ... + n_{p-1}, zero padding after the last one) and reducing
// that bucket exactly as the contiguous reduce-scatter does: chunk j = g / C
// folded in its order, averaged, written to rank (j - shift) mod K at g - jC.
// The bucket itself is never written: each input element is read once from its
// fragment.
//
// A launch carries a batch of fragments (their K rank pointers, offsets and
// sizes) in its kernel arguments; the padding tail is one more entry whose
// pointers are null (it reads as zeros). blockIdx.y = entry, blockIdx.x
// strides over 2048-element tiles of the entry; a lane owns 8 consecutive
// elements of the fragment. The block copies its entry's K pointers to LDS, so
// a lane can fold any chunk's ring order. Groups of 8 that lie in one chunk
// and start 16-byte aligned in every rank's fragment load 16 bytes per rank;
// their outputs are stored as one group when aligned, else element by element.
#include "zr_fold.hpp"

namespace zr {
namespace {

struct RsfArgs {
    const void* ptr[kRsfPtrsPerLaunch];  // entry-major: ptr[m * K + r]
    int64_t off[kRsfEntriesPerLaunch];   // virtual-bucket offset of entry m
    int64_t n[kRsfEntriesPerLaunch];     // elements of entry m
    MutPtrs out;
    int64_t N, C;
    int K, shift, accumulate, pad_;
    float inv_k, kf;
};

template <typename TIn, typename TOut, int AVG, int ORDER>
__global__ void __launch_bounds__(kThreads) rsf_kernel(const RsfArgs a) {
    const int K = a.K;
    const int m = blockIdx.y;
    __shared__ const void* sp[kMaxRanks];
    if (threadIdx.x == 0)
        for (int r = 0; r < K; ++r) sp[r] = a.ptr[m * K + r];
    __syncthreads();
    const bool padding = sp[0] == nullptr;
    auto ptr = [&](int r) { return sp[r]; };
    const int64_t n = a.n[m], off = a.off[m], C = a.C;
    const int64_t tiles = (n + kTile - 1) / kTile;

    // one output element at virtual index g (fragment-local l)
    auto elem = [&](int64_t l, int64_t g, int j) {
        float s = 0.0f;
        if (!padding) {
            s = fold_elem<TIn, ORDER>(ptr, K, j, l);
            s = average<AVG>(s, a.inv_k, a.kf);
        }
        TOut* o = static_cast<TOut*>(a.out.p[wrap(j - a.shift + K, K)]) + (g - (int64_t)j * C);
        if (a.accumulate) s = __fadd_rn(load_elem(o), s);
        store_elem(o, s);
    };

    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t l0 = t * kTile + (int64_t)threadIdx.x * kGroup;
        if (l0 >= n) continue;
        const int64_t g0 = off + l0;
        const int j0 = (int)(g0 / C);
        const int cnt = (int)((n - l0) < kGroup ? (n - l0) : kGroup);
        const bool one_chunk = (g0 + cnt - 1) < (int64_t)(j0 + 1) * C;
        bool aligned = !padding && cnt == kGroup && one_chunk;
        if (aligned)
            for (int r = 0; r < K; ++r)
                aligned = aligned && ((uintptr_t)(static_cast<const TIn*>(sp[r]) + l0) & 15) == 0;
        if (aligned) {
            // ring / wire / free order over 16-byte groups, pointers from LDS
            float acc[8];
            if constexpr (ORDER == kFree) {
                widen(load_group<TIn, false>(static_cast<const TIn*>(sp[0]) + l0), acc);
                for (int r = 1; r < K; ++r) {
                    float f[8];
                    widen(load_group<TIn, false>(static_cast<const TIn*>(sp[r]) + l0), f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = __fadd_rn(acc[e], f[e]);
                }
            } else {
                widen(load_group<TIn, false>(static_cast<const TIn*>(sp[j0]) + l0), acc);
                int r = j0;
                for (int h = 1; h < K; ++h) {
                    r = wrap(r + 1, K);
                    float f[8];
                    widen(load_group<TIn, false>(static_cast<const TIn*>(sp[r]) + l0), f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        acc[e] = __fadd_rn(acc[e], f[e]);
                        if constexpr (ORDER == kWire) acc[e] = wire_round(acc[e]);
                    }
                }
            }
            TOut* o = static_cast<TOut*>(a.out.p[wrap(j0 - a.shift + K, K)]) + (g0 - (int64_t)j0 * C);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = average<AVG>(acc[e], a.inv_k, a.kf);
            if (((uintptr_t)o & 15) == 0) {
                if (a.accumulate) {
                    float old[8];
                    widen(load_group<TOut, false>(o), old);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = __fadd_rn(old[e], acc[e]);
                }
                store_group<TOut, false>(o, pack<TOut>(acc));
            } else {
                for (int e = 0; e < 8; ++e) {
                    float s = acc[e];
                    if (a.accumulate) s = __fadd_rn(load_elem(o + e), s);
                    store_elem(o + e, s);
                }
            }
        } else {
            for (int e = 0; e < cnt; ++e) {
                const int64_t g = g0 + e;
                elem(l0 + e, g, (int)(g / C));
            }
        }
    }
}

template <typename TIn, typename TOut, int AVG, int ORDER>
hipError_t launch_t(const RsfArgs& a, int entries, int64_t max_tiles, hipStream_t stream) {
    int64_t want = (int64_t)device_cu_count() * 8 / entries;
    if (want < 1) want = 1;
    const int gx = (int)(want < max_tiles ? want : max_tiles);
    hipLaunchKernelGGL((rsf_kernel<TIn, TOut, AVG, ORDER>), dim3(gx, entries), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut, int AVG>
hipError_t pick_order(const RsfArgs& a, int entries, int64_t mt, int order, hipStream_t s) {
    if (order == kFree) return launch_t<TIn, TOut, AVG, kFree>(a, entries, mt, s);
    if (order == kWire && sizeof(TIn) == 2) return launch_t<TIn, TOut, AVG, kWire>(a, entries, mt, s);
    return launch_t<TIn, TOut, AVG, kRing>(a, entries, mt, s);
}

template <typename TIn, typename TOut>
hipError_t pick_avg(const RsfArgs& a, int entries, int64_t mt, int avg, int order, hipStream_t s) {
    switch (avg) {
        case 1: return pick_order<TIn, TOut, 1>(a, entries, mt, order, s);
        case 2: return pick_order<TIn, TOut, 2>(a, entries, mt, order, s);
        default: return pick_order<TIn, TOut, 0>(a, entries, mt, order, s);
    }
}

}  // namespace

hipError_t launch_reduce_scatter_frags(int K, const FragEntry* entries, int n_entries, int64_t N,
                                       zr_dtype in_dt, const MutPtrs& out, zr_dtype out_dt,
                                       int shift, int flags, zr_order order, hipStream_t stream) {
    RsfArgs a;
    a.out = out;
    a.N = N;
    a.K = K;
    a.C = (N + K - 1) / K;
    a.shift = shift;
    a.accumulate = (flags & ZR_ACCUMULATE) ? 1 : 0;
    a.pad_ = 0;
    a.inv_k = 1.0f / (float)K;
    a.kf = (float)K;
    const bool pow2 = (K & (K - 1)) == 0;
    const int avg = !(flags & ZR_AVERAGE) ? 0 : (pow2 ? 1 : 2);
    const int ord = order == ZR_ORDER_FREE ? kFree : (order == ZR_ORDER_RING_WIRE ? kWire : kRing);
    // entries per launch: bounded by the entry slots and by the pointer slots
    const int per = (kRsfPtrsPerLaunch / K) < kRsfEntriesPerLaunch ? (kRsfPtrsPerLaunch / K)
                                                                   : kRsfEntriesPerLaunch;
    for (int e0 = 0; e0 < n_entries; e0 += per) {
        const int cnt = (n_entries - e0) < per ? (n_entries - e0) : per;
        int64_t max_tiles = 1;
        for (int m = 0; m < cnt; ++m) {
            const FragEntry& f = entries[e0 + m];
            a.off[m] = f.off;
            a.n[m] = f.n;
            for (int r = 0; r < K; ++r) a.ptr[m * K + r] = f.ptr[r];
            const int64_t t = (f.n + kTile - 1) / kTile;
            if (t > max_tiles) max_tiles = t;
        }
        hipError_t e;
        if (in_dt == ZR_BF16 && out_dt == ZR_FP32)
            e = pick_avg<uint16_t, float>(a, cnt, max_tiles, avg, ord, stream);
        else if (in_dt == ZR_BF16 && out_dt == ZR_BF16)
            e = pick_avg<uint16_t, uint16_t>(a, cnt, max_tiles, avg, ord, stream);
        else if (in_dt == ZR_FP32 && out_dt == ZR_FP32)
            e = pick_avg<float, float>(a, cnt, max_tiles, avg, ord, stream);
        else
            e = pick_avg<float, uint16_t>(a, cnt, max_tiles, avg, ord, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zr
