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
//
// When the bases sit in different quad phases (views that start a different
// number of elements past a quad boundary in each rank), the tiles lie on
// rank 0's input lines, every input quad is read as the two aligned quads
// holding it and joined in registers, and each wave's results go through LDS:
// every rank reads back the quads aligned to its own output and stores them
// whole, its at most 3 + 3 edge elements one by one. (Element-by-element
// folds of such views ran 2.3-5.8x slower at K = 8-64.)
#include "zr_fold_any.hpp"

namespace zr {
namespace {

struct ArArgs {
    ConstPtrs in;
    MutPtrs out;
    int64_t N, C, n_tiles;
    int64_t lead;  // tiles start at this global index (< 64): quads aligned in every buffer
    int K;
    int vec;  // every in/out base the same `lead` elements before a quad boundary
    int any;  // bases in different quad phases: tiles start on rank 0's input lines
    float inv_k, kf;
};

template <typename T>
constexpr int kArSlices = sizeof(T) == 2 ? 8 : 4;  // 16 KiB of output per rank per tile
template <typename T>
constexpr int64_t kArTile = (int64_t)(kThreads / 64) * kArSlices<T> * 256;

// One tile of a launch whose bases sit in different quad phases: tile
// [t0, t1), t0 on rank 0's quad grid. Every lane folds its quad of each
// slice (whole quads below N inside one chunk as joined quads, in its own
// chunk's ring order; the rest element by element), the wave writes its
// span of S * 256 results to LDS, and each rank's output then takes the
// aligned quads of its own grid from there: span index p = 256k + 4 lane +
// sh_r, with sh_r = 4 - (its phase), plus its sh_r leading and 4 - sh_r
// trailing elements one by one (lanes 0 and 63). Stores stop at N. All loads
// of the tile precede the block barrier before the first store, so in-place
// calls read every input before it is overwritten.
template <typename T, int KS, int AVG, int ORDER, bool NT, int S, typename PtrFn>
__device__ __forceinline__ void ar_tile_any(const ArArgs& a, PtrFn lds_ptr, T (*stage)[S * 256], int64_t t0,
                                            int64_t t1) {
    constexpr int64_t TT = (int64_t)(kThreads / 64) * S * 256;
    constexpr bool WIRE = ORDER == kWire;
    const int K = KS > 0 ? KS : a.K;
    const int64_t N = a.N, C = a.C;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t span0 = t0 + (int64_t)wave * (S * 256);  // the wave's first index
    const int64_t g0 = span0 + lane * 4;
    const int j0 = (int)(t0 / C);
    T* st = stage[wave];
    auto put = [&](int k, const float (&acc)[4]) __attribute__((always_inline)) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = average<AVG>(acc[e], a.inv_k, a.kf);
        const Quad<T> q = pack4<T>(v);
        // the quad's four results, in element order, into the wave's span
        T* d = st + 256 * k + 4 * lane;
        if constexpr (sizeof(T) == 2) {
            d[0] = (T)(q.v.x & 0xFFFFu);
            d[1] = (T)(q.v.x >> 16);
            d[2] = (T)(q.v.y & 0xFFFFu);
            d[3] = (T)(q.v.y >> 16);
        } else {
            d[0] = q.v.x;
            d[1] = q.v.y;
            d[2] = q.v.z;
            d[3] = q.v.w;
        }
    };
    if ((int)((t1 - 1) / C) == j0 && t1 - t0 == TT) {
        // inside one chunk and below N: the chunk (hence the ranks' order) is
        // uniform, so each rank's phase and base stay scalar
        float acc[S][4];
        auto ptr = [&](int r) { return a.in.p[r]; };
        if constexpr (ORDER == kFree)
            fold_free_quads_any<T, KS, NT, S>(ptr, K, g0, t0, acc);
        else
            fold_ring_quads_any<T, KS, NT, S, WIRE>(ptr, K, j0, g0, t0, acc);
#pragma unroll
        for (int k = 0; k < S; ++k) put(k, acc[k]);
    } else {
#pragma unroll 1
        for (int k = 0; k < S; ++k) {
            const int64_t q = g0 + 256 * k;  // this lane's quad in slice k
            const int jq = (int)(q / C);
            if (q + 4 <= N && (q + 3) / C == jq) {
                float acc[1][4];
                if constexpr (ORDER == kFree)
                    fold_free_quads_any<T, KS, NT, 1>(lds_ptr, K, q, t0, acc);
                else
                    fold_ring_quads_any<T, KS, NT, 1, WIRE>(lds_ptr, K, jq, q, t0, acc);
                put(k, acc[0]);
                continue;
            }
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int e = 0; e < 4; ++e)
                if (q + e < N) acc[e] = fold_elem<T, KS, ORDER>(lds_ptr, K, (int)((q + e) / C), q + e);
            put(k, acc);
        }
    }
    __syncthreads();  // every wave's loads are done and its span is staged
    for (int r = 0; r < K; ++r) {
        T* out = static_cast<T*>(a.out.p[r]) + span0;
        // elements from the wave's span start to rank r's next quad boundary
        const int sh = (int)(((4 * sizeof(T) - (uintptr_t)out % (4 * sizeof(T))) % (4 * sizeof(T))) / sizeof(T));
#pragma unroll
        for (int k = 0; k < S; ++k) {
            const int p = 256 * k + 4 * lane + sh;
            if (p + 4 > S * 256) continue;  // lane 63 of the last slice: the tail
            const int64_t g = span0 + p;
            T v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = st[p + e];
            if (g + 4 <= N) {
                Quad<T> q;
                if constexpr (sizeof(T) == 2)
                    q.v = u32x2{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
                else
                    q.v = f32x4{v[0], v[1], v[2], v[3]};
                store_quad<T, NT>(out + p, q);
            } else {
                for (int e = 0; e < 4; ++e)
                    if (g + e < N) out[p + e] = v[e];
            }
        }
        if (lane == 0)
            for (int e = 0; e < sh; ++e)
                if (span0 + e < N) out[e] = st[e];
        if (lane == 63)
            for (int e = S * 256 - 4 + sh; e < S * 256; ++e)
                if (sh > 0 && span0 + e < N) out[e] = st[e];
    }
    __syncthreads();  // the stage is read before the next tile writes it
}

template <typename T, int KS, int AVG, int ORDER, bool NT, bool ANY>
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
    if constexpr (ANY) {
        __shared__ T stage[kThreads / 64][S * 256];
        for (int64_t t = blockIdx.x; t < a.n_tiles; t += gridDim.x) {
            const int64_t t0 = a.lead + t * TT;
            ar_tile_any<T, KS, AVG, ORDER, NT, S>(a, lds_ptr, stage, t0, (t0 + TT < N) ? t0 + TT : N);
        }
    } else {
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
}

template <typename T, int KS, int AVG, int ORDER, bool NT, bool ANY = false>
hipError_t launch_t(const ArArgs& a, hipStream_t stream) {
    // one block per tile; at least one, which also folds the elements before the tiles
    const int gx = a.n_tiles > 0 ? grid_for(a.n_tiles) : 1;
    hipLaunchKernelGGL((ar_kernel<T, KS, AVG, ORDER, NT, ANY>), dim3(gx), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int KS, int AVG, int ORDER, bool ANY = false>
hipError_t pick_nt(const ArArgs& a, hipStream_t s) {
    return tuning().ar_nontemporal ? launch_t<T, KS, AVG, ORDER, true, ANY>(a, s)
                                   : launch_t<T, KS, AVG, ORDER, false, ANY>(a, s);
}

template <typename T, int AVG>
hipError_t pick_k(const ArArgs& a, int order, hipStream_t s) {
    if (a.any) {  // bases in different quad phases: the generic kernels built for them
        if (order == kFree) return pick_nt<T, 0, AVG, kFree, true>(a, s);
        if (order == kWire && sizeof(T) == 2) return pick_nt<T, 0, AVG, kWire, true>(a, s);
        return pick_nt<T, 0, AVG, kRing, true>(a, s);
    }
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
    const int ord = order == ZR_ORDER_FREE ? kFree : (order == ZR_ORDER_RING_WIRE ? kWire : kRing);
    a.vec = vec ? 1 : 0;
    // bases in different quad phases: tiles on rank 0's input lines, every
    // quad read as an aligned pair
    a.any = !vec && tuning().force_path != kPathElement ? 1 : 0;
    a.lead = a.any ? (int64_t)(((128 - line_phase) % 128) / es)
                   : !vec ? 0 : (int64_t)((same_line ? (128 - line_phase) % 128 : (al - phase) % al) / es);
    if (a.lead > N) a.lead = N;
    a.n_tiles = (N - a.lead + tile - 1) / tile;
    const bool pow2 = (K & (K - 1)) == 0;
    const int avg_mode = !average ? 0 : (pow2 ? 1 : 2);
    if (dt == ZR_BF16) return pick_avg<uint16_t>(a, avg_mode, ord, stream);
    return pick_avg<float>(a, avg_mode, ord, stream);
}

}  // namespace zr
