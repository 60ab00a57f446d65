// Per-lane folds over K rank buffers, shared by the reduce-scatter and the
// fused all-reduce kernels.
//
// Ring order (the path a chunk takes around the ring, "图解 Ring All-Reduce",
// Phase 1): chunk j starts with rank j's value and adds ranks j+1, ..., j-1
// (mod K), one fp32 add per hop, so the result is
//     (((x_j + x_{j+1}) + x_{j+2}) + ... ) + x_{j-1}.
// The fold keeps up to eight ranks' 16-byte loads in flight per lane, then
// adds them strictly in that order: the loads may be issued in any order,
// the adds may not.
//
// Free order: ranks 0..K-1 in batches of eight, each batch summed as a
// balanced pairwise tree, batches added in sequence. Not bit-identical to the
// ring order; within the fp32 summation error bound of the exact sum.
//
// Wire order: the ring order with every hop's partial sum rounded to bf16
// before the next hop adds to it, as a ring that carries bf16 partial sums
// between ranks does (the receiver adds in fp32 and sends on a bf16 value).
#pragma once

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
// whole kernel when K is a small compile-time constant.
template <typename TIn, int KS>
struct RingBases {
    const TIn* p[KS];
    __device__ __forceinline__ RingBases(const ConstPtrs& in, int j) {
#pragma unroll
        for (int h = 0; h < KS; ++h) p[h] = static_cast<const TIn*>(in.p[wrap(j + h, KS)]);
    }
};

// Ring-order fold of the 8-element group at global index g (16-byte aligned
// in every rank buffer), K = KS <= 16 known at compile time: all K loads are
// issued before the first add (the scheduling barrier keeps the compiler
// from waiting on the first load early), then the adds run in ring order.
template <typename TIn, int KS, bool NT>
__device__ __forceinline__ void fold_ring_group_static(const RingBases<TIn, KS>& b, int64_t g,
                                                       float acc[8]) {
    Group<TIn> v[KS];
#pragma unroll
    for (int h = 0; h < KS; ++h) v[h] = load_group<TIn, NT>(b.p[h] + g);
    __builtin_amdgcn_sched_barrier(0);
    widen(v[0], acc);
#pragma unroll
    for (int h = 1; h < KS; ++h) accumulate(acc, v[h]);
}

// Ring-order fold for any K: batches of eight ranks' loads in flight, folded
// in ring order batch after batch. `in.p[...]` is indexed with block-uniform
// values, so the pointers come from scalar loads.
template <typename TIn, int KS, bool NT>
__device__ __forceinline__ void fold_ring_group(const ConstPtrs& in, int K, int j, int64_t g,
                                                float acc[8]) {
    constexpr int B = 8;
    const int Kr = KS > 0 ? KS : K;
    for (int h0 = 0; h0 < Kr; h0 += B) {
        Group<TIn> v[B];
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (h0 + b < Kr)
                v[b] = load_group<TIn, NT>(static_cast<const TIn*>(in.p[wrap(j + h0 + b, Kr)]) + g);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (h0 + b < Kr) {
                if (h0 + b == 0)
                    widen(v[b], acc);
                else
                    accumulate(acc, v[b]);
            }
        }
    }
}

// Free-order fold of a group (pairwise within batches of eight ranks).
template <typename TIn, int KS, bool NT>
__device__ __forceinline__ void fold_free_group(const ConstPtrs& in, int K, int64_t g,
                                                float acc[8]) {
    constexpr int B = 8;
    const int Kr = KS > 0 ? KS : K;
    for (int h0 = 0; h0 < Kr; h0 += B) {
        float f[B][8];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (h0 + b < Kr) {
                widen(load_group<TIn, NT>(static_cast<const TIn*>(in.p[h0 + b]) + g), f[b]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) f[b][e] = 0.0f;
            }
        }
#pragma unroll
        for (int s = 1; s < B; s *= 2)
#pragma unroll
            for (int b = 0; b + s < B; b += 2 * s)
                if (h0 + b + s < Kr)
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[b][e] = __fadd_rn(f[b][e], f[b + s][e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = (h0 == 0) ? f[0][e] : __fadd_rn(acc[e], f[0][e]);
    }
}

// ------------------------------------------------------------------ quads
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

// Ring order for any K: batches of eight ranks, every slice's loads of a batch
// in flight together, batches folded in ring order one after the other.
template <typename TIn, int KS, bool NT, int S, bool WIRE = false>
__device__ __forceinline__ void fold_ring_quads(const ConstPtrs& in, int K, int j, int64_t g0,
                                                float acc[S][4]) {
    constexpr int B = 8;
    const int Kr = KS > 0 ? KS : K;
    for (int h0 = 0; h0 < Kr; h0 += B) {
        Quad<TIn> v[S][B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (h0 + b < Kr) {
                const TIn* p = static_cast<const TIn*>(in.p[wrap(j + h0 + b, Kr)]);
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
template <typename TIn, int KS, bool NT, int S>
__device__ __forceinline__ void fold_free_quads(const ConstPtrs& in, int K, int64_t g0,
                                                float acc[S][4]) {
    constexpr int B = 8;
    const int Kr = KS > 0 ? KS : K;
    for (int h0 = 0; h0 < Kr; h0 += B) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
            float f[B][4];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (h0 + b < Kr) {
                    widen4(load_quad<TIn, NT>(static_cast<const TIn*>(in.p[h0 + b]) + g0 + 256 * k), f[b]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) f[b][e] = 0.0f;
                }
            }
#pragma unroll
            for (int s = 1; s < B; s *= 2)
#pragma unroll
                for (int b = 0; b + s < B; b += 2 * s)
                    if (h0 + b + s < Kr)
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[b][e] = __fadd_rn(f[b][e], f[b + s][e]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[k][e] = (h0 == 0) ? f[0][e] : __fadd_rn(acc[k][e], f[0][e]);
        }
    }
}

// Scalar ring-order fold of one element (index g < N) of chunk j, with the
// rank pointers read through `ptr(r)` (kernel arguments or an LDS table).
template <typename TIn, typename PtrFn, bool WIRE = false>
__device__ __forceinline__ float fold_ring_elem(PtrFn ptr, int K, int j, int64_t g) {
    float acc = load_elem(static_cast<const TIn*>(ptr(j)) + g);
    int r = j;
    for (int h = 1; h < K; ++h) {
        r = wrap(r + 1, K);
        acc = __fadd_rn(acc, load_elem(static_cast<const TIn*>(ptr(r)) + g));
        if constexpr (WIRE) acc = wire_round(acc);
    }
    return acc;
}


// Scalar free-order fold (ranks in index order).
template <typename TIn, typename PtrFn>
__device__ __forceinline__ float fold_free_elem(PtrFn ptr, int K, int64_t g) {
    float acc = load_elem(static_cast<const TIn*>(ptr(0)) + g);
    for (int r = 1; r < K; ++r) acc = __fadd_rn(acc, load_elem(static_cast<const TIn*>(ptr(r)) + g));
    return acc;
}

// A wave's S quads in the given order; kStatic uses the bases held in scalar
// registers (ring or wire order, K = KS <= 8).
template <typename TIn, int KS, bool NT, int S, int ORDER, bool kStatic>
__device__ __forceinline__ void fold_quads(const RingBases<TIn, kStatic ? KS : 1>& bases,
                                           const ConstPtrs& in, int K, int j, int64_t g0,
                                           float acc[S][4]) {
    if constexpr (ORDER == kFree)
        fold_free_quads<TIn, KS, NT, S>(in, K, g0, acc);
    else if constexpr (kStatic)
        fold_ring_quads_static<TIn, KS, NT, S, ORDER == kWire>(bases, g0, acc);
    else
        fold_ring_quads<TIn, KS, NT, S, ORDER == kWire>(in, K, j, g0, acc);
}

// One element in the given order (ring, free or wire).
template <typename TIn, int ORDER, typename PtrFn>
__device__ __forceinline__ float fold_elem(PtrFn ptr, int K, int j, int64_t g) {
    if constexpr (ORDER == kFree) return fold_free_elem<TIn>(ptr, K, g);
    return fold_ring_elem<TIn, PtrFn, ORDER == kWire>(ptr, K, j, g);
}

}  // namespace zr
