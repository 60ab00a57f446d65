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
// Grid: blockIdx.y = chunk j (so j, the holder and every rank pointer are
// uniform per block), blockIdx.x strides over 2048-element tiles of the
// chunk. Each lane owns 8 consecutive outputs: one 16-byte load per rank for
// bf16 input, two 16-byte stores for fp32 output. A chunk whose input start
// j*C is not 16-byte aligned, and the ragged tail of the last chunk, take the
// element-wise path; positions g >= N are padding and receive +0.
#include "zr_fold.hpp"

namespace zr {
namespace {

struct RsArgs {
    ConstPtrs in;
    MutPtrs out;
    int64_t N, C;
    uint64_t vec_mask;  // bit j: chunk j takes the 16-byte path
    int K, shift;
    int tiles_per_chunk;
    float inv_k, kf;
};

// K small and known at compile time: the static ring fold with hoisted bases.
template <int KS>
constexpr bool kStaticFold = KS > 0 && KS <= 16;

template <typename TIn, typename TOut, int KS, int AVG, bool RING, bool NT>
__global__ void __launch_bounds__(kThreads) rs_kernel(const RsArgs a) {
    const int K = KS > 0 ? KS : a.K;
    const int j = blockIdx.y;
    const int holder = wrap(j - a.shift + K, K);
    const bool vec = (a.vec_mask >> j) & 1ull;
    const int64_t C = a.C, N = a.N;
    const int64_t chunk_base = (int64_t)j * C;
    TOut* outp = static_cast<TOut*>(a.out.p[holder]);
    auto ptr = [&](int r) { return a.in.p[r]; };
    constexpr int KB = kStaticFold<KS> ? KS : 1;
    const RingBases<TIn, KB> bases(a.in, kStaticFold<KS> ? j : 0);

    for (int t = blockIdx.x; t < a.tiles_per_chunk; t += gridDim.x) {
        const int64_t o = (int64_t)t * kTile + (int64_t)threadIdx.x * kGroup;
        if (o >= C) continue;
        const int64_t g = chunk_base + o;
        if (vec && o + kGroup <= C && g + kGroup <= N) {
            float acc[8];
            if constexpr (RING && kStaticFold<KS>)
                fold_ring_group_static<TIn, KS, NT>(bases, g, acc);
            else if constexpr (RING)
                fold_ring_group<TIn, KS, NT>(a.in, K, j, g, acc);
            else
                fold_free_group<TIn, KS, NT>(a.in, K, g, acc);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = average<AVG>(acc[e], a.inv_k, a.kf);
            store_group<TOut, NT>(outp + o, pack<TOut>(acc));
        } else {
            const int n_out = (int)((C - o) < kGroup ? (C - o) : kGroup);
            for (int e = 0; e < n_out; ++e) {
                const int64_t ge = g + e;
                float s = 0.0f;
                if (ge < N) {
                    s = RING ? fold_ring_elem<TIn>(ptr, K, j, ge) : fold_free_elem<TIn>(ptr, K, ge);
                    s = average<AVG>(s, a.inv_k, a.kf);
                }
                store_elem(outp + o + e, s);
            }
        }
    }
}

template <typename TIn, typename TOut, int KS, int AVG, bool RING, bool NT>
hipError_t launch_t(const RsArgs& a, hipStream_t stream) {
    const int cus = device_cu_count();
    int64_t want = (int64_t)cus * tuning().rs_blocks_per_cu / a.K;
    if (want < 1) want = 1;
    const int gx = (int)(want < a.tiles_per_chunk ? want : a.tiles_per_chunk);
    hipLaunchKernelGGL((rs_kernel<TIn, TOut, KS, AVG, RING, NT>), dim3(gx, a.K), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut, int KS, int AVG, bool RING>
hipError_t pick_nt(const RsArgs& a, hipStream_t s) {
    return tuning().nontemporal ? launch_t<TIn, TOut, KS, AVG, RING, true>(a, s)
                                : launch_t<TIn, TOut, KS, AVG, RING, false>(a, s);
}

template <typename TIn, typename TOut, int AVG>
hipError_t pick_k(const RsArgs& a, bool ring, hipStream_t s) {
    if (!ring) return pick_nt<TIn, TOut, 0, AVG, false>(a, s);
    switch (a.K) {
        case 8: return pick_nt<TIn, TOut, 8, AVG, true>(a, s);
        case 64: return pick_nt<TIn, TOut, 64, AVG, true>(a, s);
        default: return pick_nt<TIn, TOut, 0, AVG, true>(a, s);
    }
}

template <typename TIn, typename TOut>
hipError_t pick_avg(const RsArgs& a, int avg_mode, bool ring, hipStream_t s) {
    switch (avg_mode) {
        case 1: return pick_k<TIn, TOut, 1>(a, ring, s);
        case 2: return pick_k<TIn, TOut, 2>(a, ring, s);
        default: return pick_k<TIn, TOut, 0>(a, ring, s);
    }
}

}  // namespace

hipError_t launch_reduce_scatter(int K, const ConstPtrs& in, zr_dtype in_dt, int64_t N,
                                 const MutPtrs& out, zr_dtype out_dt, int shift, int average,
                                 zr_order order, hipStream_t stream) {
    RsArgs a;
    a.in = in;
    a.out = out;
    a.N = N;
    a.K = K;
    a.C = (N + K - 1) / K;
    a.shift = shift;
    a.tiles_per_chunk = (int)((a.C + kTile - 1) / kTile);
    a.inv_k = 1.0f / (float)K;
    a.kf = (float)K;
    const int in_es = in_dt == ZR_BF16 ? 2 : 4;
    bool bases = true;
    for (int r = 0; r < K; ++r) {
        bases = bases && (((uintptr_t)in.p[r]) & 15) == 0;
        bases = bases && (((uintptr_t)out.p[r]) & 15) == 0;
    }
    a.vec_mask = 0;
    for (int j = 0; j < K; ++j)
        if (bases && ((a.C * j * in_es) & 15) == 0) a.vec_mask |= 1ull << j;
    const bool pow2 = (K & (K - 1)) == 0;
    const int avg_mode = !average ? 0 : (pow2 ? 1 : 2);
    const bool ring = order == ZR_ORDER_RING;
    if (in_dt == ZR_BF16 && out_dt == ZR_FP32) return pick_avg<uint16_t, float>(a, avg_mode, ring, stream);
    if (in_dt == ZR_BF16 && out_dt == ZR_BF16) return pick_avg<uint16_t, uint16_t>(a, avg_mode, ring, stream);
    if (in_dt == ZR_FP32 && out_dt == ZR_FP32) return pick_avg<float, float>(a, avg_mode, ring, stream);
    return pick_avg<float, uint16_t>(a, avg_mode, ring, stream);
}

}  // namespace zr
