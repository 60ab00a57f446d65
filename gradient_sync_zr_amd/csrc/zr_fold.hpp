// Per-lane folds over K rank buffers, shared by the reduce-scatter kernels
// (contiguous and discrete) and the fused all-reduce kernel.
//
// Ring order (the path a chunk takes around the ring, "图解 Ring All-Reduce",
// Phase 1): chunk j starts with rank j's value and adds ranks j+1, ..., j-1
// (mod K), one fp32 add per hop, so the result is
//     (((x_j + x_{j+1}) + x_{j+2}) + ... ) + x_{j-1}.
// The fold keeps up to eight ranks' loads of every slice in flight per lane,
// then adds them strictly in that order: the loads may be issued in any
// order, the adds may not.
//
// Free order: ranks 0..K-1 in batches of eight, each batch summed as a
// balanced pairwise tree, batches added in sequence. Not bit-identical to the
// ring order; within the fp32 summation error bound of the exact sum.
//
// Wire order: the ring order with every hop's partial sum rounded to bf16
// before the next hop adds to it, as a ring that carries bf16 partial sums
// between ranks does (the receiver adds in fp32 and sends on a bf16 value).
#pragma once

#include <type_traits>

#include "zr_device.hpp"
#include "zr_internal.hpp"

namespace zr {

__device__ __forceinline__ int wrap(int r, int K) { return r >= K ? r - K : r; }

// Fold orders (template arguments of the kernels).
constexpr int kRing = 0;
constexpr int kFree = 1;
constexpr int kWire = 2;

// The fp32 value of v rounded to bf16 (nearest even), used between hops of
// the wire order.
__device__ __forceinline__ float wire_round(float v) { return __uint_as_float(bf16_round(v) << 16); }

template <bool WIRE>
__device__ __forceinline__ void hop4(float acc[4], const float f[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        acc[e] = __fadd_rn(acc[e], f[e]);
        if constexpr (WIRE) acc[e] = wire_round(acc[e]);
    }
}

// Rank buffers in ring order for chunk j, held in scalar registers for the
// whole tile when K is a small compile-time constant. `ptr(r)` returns rank
// r's base pointer (a kernel-argument table indexed with block-uniform
// values, so the pointers come from scalar loads).
template <typename TIn, int KS>
struct RingBases {
    const TIn* p[KS];
    template <typename PtrFn>
    __device__ __forceinline__ RingBases(PtrFn ptr, int j) {
#pragma unroll
        for (int h = 0; h < KS; ++h) p[h] = static_cast<const TIn*>(ptr(wrap(j + h, KS)));
    }
};

// ------------------------------------------------------------------ quads
// Slices per wave of the full reduce-scatter tiles (4 waves x S x 256
// elements): a tile writes 16 KiB of output, which streamed better than 8 KiB
// (bf16 -> bf16 by 5%, fp32 -> fp32 by 4%), except fp32 input with bf16 output,
// which keeps 2 slices (4 measured no faster). One-slice tiles (kRsTileOf<1>)
// serve small launches and the shapes that stream faster with them
// (ring_one_slice in the reduce-scatter's launch code lists those).
template <typename TIn, typename TOut>
constexpr int kSlices = sizeof(TOut) == 4 ? 4 : (sizeof(TIn) == 2 ? 8 : 2);
// Non-temporal (streaming) loads and stores in the reduce-scatter kernels:
// every byte is touched once, so caching it only evicts other lines.
#ifndef ZR_RS_NONTEMPORAL
#define ZR_RS_NONTEMPORAL 1
#endif
constexpr bool kRsNontemporal = ZR_RS_NONTEMPORAL != 0;
// Elements per reduce-scatter tile of S slices: 4 waves x S x 256. Ring-order
// launches too small to give every CU two tiles use one slice per wave (four
// times as many, shorter tiles).
template <int S>
constexpr int64_t kRsTileOf = (int64_t)(kThreads / 64) * S * 256;
template <typename TIn, typename TOut>
constexpr int64_t kRsTile = kRsTileOf<kSlices<TIn, TOut>>;
// Slices per wave of the generic-K kernels in the free and bf16-wire orders,
// and of the discrete kernels for ranks in different phases: at most four
// (bf16 in and out would take eight, where the generic kernels needed
// 236-256 VGPRs, ran one wave per SIMD and reached 2.4-4.5 TB/s, and the
// different-phase kernels ran 4-17% slower at K <= 16).
template <typename TIn, typename TOut>
constexpr int kSlicesGeneric = kSlices<TIn, TOut> > 4 ? 4 : kSlices<TIn, TOut>;
// Does a reduce-scatter launch at this K and fold order run those kernels?
// (The free order always does; the wire order does with bf16 input and
// K != 8, the one K it specialises.)
template <typename TIn>
__host__ __device__ constexpr bool rs_generic_narrow(int K, int order) {
    return order == kFree || (order == kWire && sizeof(TIn) == 2 && K != 8);
}

// A wave owns S slices of 256 consecutive elements; lane l holds quad l of
// each slice (elements 4l..4l+3), so every load and store instruction of the
// wave covers one contiguous span. g0 is the lane's first element; slice k
// is at g0 + 256*k.

// Ring order with K = KS <= 8 known at compile time: all S*KS loads are issued
// before the first add, then each slice is folded in ring order.
template <typename TIn, int KS, bool NT, int S, bool WIRE = false>
__device__ __forceinline__ void fold_ring_quads_static(const RingBases<TIn, KS>& b, int64_t g0,
                                                       float acc[S][4]) {
    Quad<TIn> v[S][KS];
#pragma unroll
    for (int k = 0; k < S; ++k)
#pragma unroll
        for (int h = 0; h < KS; ++h) v[k][h] = load_quad<TIn, NT>(b.p[h] + g0 + 256 * k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < S; ++k) {
        widen4(v[k][0], acc[k]);
#pragma unroll
        for (int h = 1; h < KS; ++h) {
            float f[4];
            widen4(v[k][h], f);
            hop4<WIRE>(acc[k], f);
        }
    }
}

// Ranks per batch of the ring fold for any K: the batch's loads of all S
// slices are in flight together, about 64 VGPRs of data per lane (bf16 quads
// take 2 VGPRs, fp32 quads 4), and never fewer than eight ranks. A tile of one
// or two slices thus waits on K / 32 or K / 16 round trips to memory instead of
// K / 8, which is what a launch with few tiles per CU (large K, a small bucket)
// is bound by.
template <typename TIn, int S>
constexpr int kRingBatch = (64 / (S * (int)sizeof(TIn))) > 8 ? 64 / (S * (int)sizeof(TIn)) : 8;
// The wire order keeps four ranks per batch: its per-hop rounding needs
// registers of its own, and with eight ranks the generic kernels ran at two
// waves per SIMD and 4.7-4.9 TB/s, with four at three and 5.6-6.2 TB/s
// (bf16 in, fp32 out).
constexpr int kWireBatch = 4;

// Ring order for any K: batches of kRingBatch ranks, every slice's loads of a
// batch in flight together, batches folded in ring order one after the other.
template <typename TIn, int KS, bool NT, int S, bool WIRE = false, typename PtrFn>
__device__ __forceinline__ void fold_ring_quads(PtrFn ptr, int K, int j, int64_t g0,
                                                float acc[S][4]) {
    constexpr int B = WIRE ? kWireBatch : kRingBatch<TIn, S>;
    const int Kr = KS > 0 ? KS : K;
    for (int h0 = 0; h0 < Kr; h0 += B) {
        Quad<TIn> v[S][B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (h0 + b < Kr) {
                const TIn* p = static_cast<const TIn*>(ptr(wrap(j + h0 + b, Kr)));
#pragma unroll
                for (int k = 0; k < S; ++k) v[k][b] = load_quad<TIn, NT>(p + g0 + 256 * k);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (h0 + b < Kr) {
#pragma unroll
                for (int k = 0; k < S; ++k) {
                    if (h0 + b == 0) {
                        widen4(v[k][b], acc[k]);
                    } else {
                        float f[4];
                        widen4(v[k][b], f);
                        hop4<WIRE>(acc[k], f);
                    }
                }
            }
        }
    }
}

// Free order: ranks 0..K-1 in batches of eight, pairwise within a batch.
// A batch's loads of every slice are in flight together before its trees
// (loading and consuming one rank at a time waited on a memory round trip per
// load: 2.3-5.3 TB/s with bf16 input, against 5.3-6.3 for the ring order).
template <typename TIn, int KS, bool NT, int S, typename PtrFn>
__device__ __forceinline__ void fold_free_quads(PtrFn ptr, int K, int64_t g0, float acc[S][4]) {
    constexpr int B = 8;
    const int Kr = KS > 0 ? KS : K;
    for (int h0 = 0; h0 < Kr; h0 += B) {
        Quad<TIn> v[S][B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (h0 + b < Kr) {
                const TIn* p = static_cast<const TIn*>(ptr(h0 + b));
#pragma unroll
                for (int k = 0; k < S; ++k) v[k][b] = load_quad<TIn, NT>(p + g0 + 256 * k);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < S; ++k) {
            // the tree's first level straight from the loaded pairs (pair p
            // sums ranks h0 + 2p and h0 + 2p + 1), so only half the batch is
            // held widened: the generic kernel then fits three waves per SIMD
            float f[B / 2][4];
#pragma unroll
            for (int q = 0; q < B / 2; ++q) {
                if (h0 + 2 * q < Kr) {
                    widen4(v[k][2 * q], f[q]);
                    if (h0 + 2 * q + 1 < Kr) {
                        float t[4];
                        widen4(v[k][2 * q + 1], t);
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[q][e] = __fadd_rn(f[q][e], t[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) f[q][e] = 0.0f;
                }
            }
            // the levels above: pair q holds the sum over ranks h0 + 2q ..
            // h0 + 2q + 1; level s adds the pair s further on, if present
#pragma unroll
            for (int s = 1; s < B / 2; s *= 2)
#pragma unroll
                for (int q = 0; q + s < B / 2; q += 2 * s)
                    if (h0 + 2 * (q + s) < Kr)
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[q][e] = __fadd_rn(f[q][e], f[q + s][e]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[k][e] = (h0 == 0) ? f[0][e] : __fadd_rn(acc[k][e], f[0][e]);
        }
    }
}

// Scalar ring-order fold of one element (index g < N) of chunk j, with the
// rank pointers read through `ptr(r)` (kernel arguments or an LDS table).
// Batches of eight ranks' loads are issued before their adds, so a lane waits
// on one memory latency per batch instead of one per rank.
template <typename TIn, int KS, bool WIRE, typename PtrFn>
__device__ __forceinline__ float fold_ring_elem(PtrFn ptr, int K, int j, int64_t g) {
    constexpr int B = 8;
    const int Kr = KS > 0 ? KS : K;
    float acc = 0.0f;
    for (int h0 = 0; h0 < Kr; h0 += B) {
        float v[B];
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (h0 + b < Kr) v[b] = load_elem(static_cast<const TIn*>(ptr(wrap(j + h0 + b, Kr))) + g);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (h0 + b < Kr) {
                if (h0 + b == 0) {
                    acc = v[b];
                } else {
                    acc = __fadd_rn(acc, v[b]);
                    if constexpr (WIRE) acc = wire_round(acc);
                }
            }
        }
    }
    return acc;
}

// Scalar free-order fold (ranks in index order, loads batched the same way).
template <typename TIn, int KS, typename PtrFn>
__device__ __forceinline__ float fold_free_elem(PtrFn ptr, int K, int64_t g) {
    constexpr int B = 8;
    const int Kr = KS > 0 ? KS : K;
    float acc = 0.0f;
    for (int h0 = 0; h0 < Kr; h0 += B) {
        float v[B];
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (h0 + b < Kr) v[b] = load_elem(static_cast<const TIn*>(ptr(h0 + b)) + g);
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (h0 + b < Kr) acc = (h0 + b == 0) ? v[b] : __fadd_rn(acc, v[b]);
    }
    return acc;
}

// A wave's S quads in the given order; kStatic uses the bases held in scalar
// registers (ring or wire order, K = KS <= 8).
template <typename TIn, int KS, bool NT, int S, int ORDER, bool kStatic, typename PtrFn>
__device__ __forceinline__ void fold_quads(const RingBases<TIn, kStatic ? KS : 1>& bases,
                                           PtrFn ptr, int K, int j, int64_t g0, float acc[S][4]) {
    if constexpr (ORDER == kFree)
        fold_free_quads<TIn, KS, NT, S>(ptr, K, g0, acc);
    else if constexpr (kStatic)
        fold_ring_quads_static<TIn, KS, NT, S, ORDER == kWire>(bases, g0, acc);
    else
        fold_ring_quads<TIn, KS, NT, S, ORDER == kWire>(ptr, K, j, g0, acc);
}

// One element in the given order (ring, free or wire); KS > 0 fixes K at
// compile time.
template <typename TIn, int KS, int ORDER, typename PtrFn>
__device__ __forceinline__ float fold_elem(PtrFn ptr, int K, int j, int64_t g) {
    if constexpr (ORDER == kFree) return fold_free_elem<TIn, KS>(ptr, K, g);
    return fold_ring_elem<TIn, KS, ORDER == kWire>(ptr, K, j, g);
}

}  // namespace zr
