// Fused all-reduce: reduce-scatter and all-gather in one pass.
//
// All-reduce is reduce-scatter followed by all-gather (CMU 11-868 lecture 14
// notes, 2.2). On one device the two phases need not meet in memory: each
// lane reads the K values of its 8 global indices, folds them in the ring
// order of the chunk they belong to ("图解 Ring All-Reduce", Phase 1), rounds
// once to the buffer dtype, and writes the same bits to all K ranks (the
// all-gather result of Phase 2, where every rank ends with identical sums).
// Output may be the input (in place): a lane writes index g only after it
// has read index g from every rank, and no other lane touches g.
//
// Tiles are 4 waves x S slices x 256 global indices, lanes on 4-element quads
// (as in the reduce-scatter kernel, so every store instruction writes one
// contiguous span), one block per tile in index order (a persistent grid
// striding over the tiles ran a few percent slower). S makes a tile write
// 16 KiB to every rank: at K = 64, 8 slices of bf16 ran 0.9% faster than 4. A tile that lies inside one chunk and below N takes the
// vector path with the chunk (hence the fold's first rank) uniform across the
// block. In a tile that straddles a chunk boundary or the end of the buffer
// (at most K of them) each lane folds its quads one slice at a time in the
// ring order of the quad's own chunk, reading the rank pointers from an LDS
// table; only a quad that a chunk boundary or the end of the buffer cuts folds
// element by element. (Folding these tiles element by element, a lane waited
// on K / 8 memory round trips per element, and the few such blocks set the
// launch time: +21-55% at K = 16-64 and 16M elements.) When every input and
// output base lies the same number of elements past a quad boundary, the tile
// grid starts where they reach the next one (`lead` elements in; the next
// 128-byte line when the bases agree within lines), so every quad is aligned;
// block 0 folds the first `lead` (< 64) elements one by one. (Such views folded
// element by element throughout ran 2.5-3.6x slower.)
#include "zr_fold.hpp"

namespace zr {
namespace {

struct ArArgs {
    ConstPtrs in;
    MutPtrs out;
    int64_t N, C, n_tiles;
    int64_t lead;  // tiles start at this global index (< 64): quads aligned in every buffer
    int K;
    int vec;  // every in/out base the same `lead` elements before a quad boundary
    float inv_k, kf;
};

template <typename T>
constexpr int kArSlices = sizeof(T) == 2 ? 8 : 4;  // 16 KiB of output per rank per tile
template <typename T>
constexpr int64_t kArTile = (int64_t)(kThreads / 64) * kArSlices<T> * 256;

template <typename T, int KS, int AVG, int ORDER, bool NT>
__global__ void __launch_bounds__(kThreads) ar_kernel(const ArArgs a) {
    constexpr int S = kArSlices<T>;
    constexpr int64_t TT = kArTile<T>;
    const int K = KS > 0 ? KS : a.K;
    __shared__ const void* s_in[kMaxRanks];
    if (threadIdx.x == 0)
        for (int r = 0; r < K; ++r) s_in[r] = a.in.p[r];
    __syncthreads();
    auto lds_ptr = [&](int r) { return s_in[r]; };
    const int64_t N = a.N, C = a.C;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    if (blockIdx.x == 0 && threadIdx.x < a.lead && threadIdx.x < N) {
        // the elements before the tile grid, one per thread
        const int64_t ge = threadIdx.x;
        float s = fold_elem<T, KS, ORDER>(lds_ptr, K, (int)(ge / C), ge);
        s = average<AVG>(s, a.inv_k, a.kf);
        T v;
        store_elem(&v, s);
        for (int r = 0; r < K; ++r) static_cast<T*>(a.out.p[r])[ge] = v;
    }
    for (int64_t t = blockIdx.x; t < a.n_tiles; t += gridDim.x) {
        const int64_t t0 = a.lead + t * TT;
        const int64_t t1 = (t0 + TT < N) ? t0 + TT : N;
        const int j0 = (int)(t0 / C);
        const int j1 = (int)((t1 - 1) / C);
        const int64_t g0 = t0 + (int64_t)wave * (S * 256) + lane * 4;
        if (a.vec && j0 == j1 && t1 - t0 == TT) {
            float acc[S][4];
            constexpr bool kStatic = ORDER != kFree && KS > 0 && KS <= 8;
            auto ptr = [&](int r) { return a.in.p[r]; };
            fold_quads<T, KS, NT, S, ORDER, kStatic>(RingBases<T, kStatic ? KS : 1>(ptr, kStatic ? j0 : 0),
                                                      ptr, K, j0, g0, acc);
            Quad<T> res[S];
#pragma unroll
            for (int k = 0; k < S; ++k) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[k][e] = average<AVG>(acc[k][e], a.inv_k, a.kf);
                res[k] = pack4<T>(acc[k]);
            }
            // the all-gather: the same bits to every rank
            for (int r = 0; r < K; ++r) {
                T* o = static_cast<T*>(a.out.p[r]) + g0;
#pragma unroll
                for (int k = 0; k < S; ++k) store_quad<T, NT>(o + 256 * k, res[k]);
            }
        } else {
#pragma unroll 1
            for (int k = 0; k < S; ++k) {
                const int64_t q = g0 + 256 * k;  // this lane's quad in slice k
                const int jq = (int)(q / C);
                if (a.vec && q + 4 <= N && (q + 3) / C == jq) {
                    float acc[1][4];
                    fold_quads<T, KS, NT, 1, ORDER, false>(RingBases<T, 1>(lds_ptr, 0), lds_ptr, K, jq, q, acc);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[0][e] = average<AVG>(acc[0][e], a.inv_k, a.kf);
                    const Quad<T> res = pack4<T>(acc[0]);
                    for (int r = 0; r < K; ++r) store_quad<T, NT>(static_cast<T*>(a.out.p[r]) + q, res);
                    continue;
                }
                for (int e = 0; e < 4; ++e) {
                    const int64_t ge = q + e;
                    if (ge >= N) continue;
                    float s = fold_elem<T, KS, ORDER>(lds_ptr, K, (int)(ge / C), ge);
                    s = average<AVG>(s, a.inv_k, a.kf);
                    T v;
                    store_elem(&v, s);
                    for (int r = 0; r < K; ++r) static_cast<T*>(a.out.p[r])[ge] = v;
                }
            }
        }
    }
}

template <typename T, int KS, int AVG, int ORDER, bool NT>
hipError_t launch_t(const ArArgs& a, hipStream_t stream) {
    // one block per tile; at least one, which also folds the elements before the tiles
    const int gx = a.n_tiles > 0 ? grid_for(a.n_tiles) : 1;
    hipLaunchKernelGGL((ar_kernel<T, KS, AVG, ORDER, NT>), dim3(gx), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int KS, int AVG, int ORDER>
hipError_t pick_nt(const ArArgs& a, hipStream_t s) {
    return tuning().ar_nontemporal ? launch_t<T, KS, AVG, ORDER, true>(a, s)
                                   : launch_t<T, KS, AVG, ORDER, false>(a, s);
}

template <typename T, int AVG>
hipError_t pick_k(const ArArgs& a, int order, hipStream_t s) {
    if (order == kFree) return pick_nt<T, 0, AVG, kFree>(a, s);
    if (order == kWire && sizeof(T) == 2) return pick_nt<T, 0, AVG, kWire>(a, s);
    switch (a.K) {
        case 8: return pick_nt<T, 8, AVG, kRing>(a, s);
        case 64: return pick_nt<T, 64, AVG, kRing>(a, s);
        default: return pick_nt<T, 0, AVG, kRing>(a, s);
    }
}

template <typename T>
hipError_t pick_avg(const ArArgs& a, int avg_mode, int order, hipStream_t s) {
    switch (avg_mode) {
        case 1: return pick_k<T, 1>(a, order, s);
        case 2: return pick_k<T, 2>(a, order, s);
        default: return pick_k<T, 0>(a, order, s);
    }
}

}  // namespace

hipError_t launch_allreduce_fused(int K, const ConstPtrs& in, const MutPtrs& out, zr_dtype dt,
                                  int64_t N, int average, zr_order order, hipStream_t stream) {
    ArArgs a;
    a.in = in;
    a.out = out;
    a.N = N;
    a.K = K;
    a.C = (N + K - 1) / K;
    a.inv_k = 1.0f / (float)K;
    a.kf = (float)K;
    const int64_t tile = dt == ZR_BF16 ? kArTile<uint16_t> : kArTile<float>;
    const uintptr_t al = dt == ZR_BF16 ? 8 : 16;  // quad size
    const uintptr_t es = dt == ZR_BF16 ? 2 : 4;
    // every base in the same phase within a quad: tiles start where that
    // phase reaches the next quad boundary
    // (within a 128-byte line when they all agree there too, so tiles also
    // start on lines and no two tiles fetch the same line)
    const uintptr_t phase = (uintptr_t)in.p[0] % al, line_phase = (uintptr_t)in.p[0] % 128;
    bool vec = tuning().force_path != kPathElement, same_line = true;
    for (int r = 0; r < K; ++r) {
        vec = vec && ((uintptr_t)in.p[r] % al) == phase && ((uintptr_t)out.p[r] % al) == phase;
        same_line = same_line && ((uintptr_t)in.p[r] % 128) == line_phase && ((uintptr_t)out.p[r] % 128) == line_phase;
    }
    a.vec = vec ? 1 : 0;
    a.lead = !vec ? 0 : (int64_t)((same_line ? (128 - line_phase) % 128 : (al - phase) % al) / es);
    if (a.lead > N) a.lead = N;
    a.n_tiles = (N - a.lead + tile - 1) / tile;
    const bool pow2 = (K & (K - 1)) == 0;
    const int avg_mode = !average ? 0 : (pow2 ? 1 : 2);
    const int ord = order == ZR_ORDER_FREE ? kFree : (order == ZR_ORDER_RING_WIRE ? kWire : kRing);
    if (dt == ZR_BF16) return pick_avg<uint16_t>(a, avg_mode, ord, stream);
    return pick_avg<float>(a, avg_mode, ord, stream);
}

}  // namespace zr
