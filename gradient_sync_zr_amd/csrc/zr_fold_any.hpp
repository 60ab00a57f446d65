// Folds over rank buffers whose quad phases differ (ring, wire and free
// orders).
//
// The quad folds of zr_fold.hpp need every rank's buffer on one quad grid:
// each lane loads a quad of every rank with one aligned access. When ranks
// sit at different phases (views that start a different number of elements
// past a quad boundary in each rank), the tile grid is laid on one rank's
// quads and every other rank r is `sig_r` bytes off it. Rank r's quad is then
// read as the two aligned quads that hold its bytes (only the first when
// sig_r = 0, so no read leaves the quad's own bytes; skipping that second
// load ran 2.5-5% faster than repeating the first) and joined in registers
// with byte-align instructions. The adds keep the ring order of
// "图解 Ring All-Reduce", Phase 1, exactly as the aligned folds do: only how
// the addends reach the registers changes.
//
// Every aligned block read holds at least one byte of the quad it serves, so
// no read leaves the pages the quad lies in.
#pragma once

#include "zr_fold.hpp"

namespace zr {

// The quad at byte phase sig (0..QB-1, a multiple of the element size)
// within the two aligned quads lo:hi.
__device__ __forceinline__ Quad<uint16_t> join_quad(const Quad<uint16_t>& lo, const Quad<uint16_t>& hi,
                                                    uint32_t sig) {
    const uint32_t b = sig & 3;
    const bool up = sig >= 4;  // the quad starts in lo's second dword
    const uint32_t w0 = up ? lo.v.y : lo.v.x;
    const uint32_t w1 = up ? hi.v.x : lo.v.y;
    const uint32_t w2 = up ? hi.v.y : hi.v.x;
    return {u32x2{__builtin_amdgcn_alignbyte(w1, w0, b), __builtin_amdgcn_alignbyte(w2, w1, b)}};
}
__device__ __forceinline__ Quad<float> join_quad(const Quad<float>& lo, const Quad<float>& hi, uint32_t sig) {
    // fp32 phases are whole dwords: select, no byte shift
    const f32x4 a = lo.v, c = hi.v;
    const uint32_t d = sig >> 2;
    f32x4 r;
    r.x = d == 0 ? a.x : (d == 1 ? a.y : (d == 2 ? a.z : a.w));
    r.y = d == 0 ? a.y : (d == 1 ? a.z : (d == 2 ? a.w : c.x));
    r.z = d == 0 ? a.z : (d == 1 ? a.w : (d == 2 ? c.x : c.y));
    r.w = d == 0 ? a.w : (d == 1 ? c.x : (d == 2 ? c.y : c.z));
    return {r};
}

// Slices whose loads one batch keeps in flight, eight ranks per batch: two
// aligned quads per rank and slice, 64 VGPRs of data per lane (as many loads
// in flight as the aligned folds keep, at a register count that leaves room
// for a few blocks per CU).
template <typename TIn, int S>
constexpr int kAnySlices = S < (sizeof(TIn) == 2 ? 2 : 1) ? S : (sizeof(TIn) == 2 ? 2 : 1);
constexpr int kAnyBatch = 8;

// Ring (or wire) order over ranks in any quad phases: acc[k] = the fold of
// the quads at element g0 + 256k, chunk j. gu is an element index congruent
// to g0 modulo 4 (it fixes each rank's phase on the tile grid). `ptr(r)`
// returns rank r's base. With j, gu and the pointers uniform over the wave,
// the phases and rank bases stay in scalar registers; a lane-varying j (a
// tile that straddles chunks) gives each lane its own ranks and phases.
template <typename TIn, int KS, bool NT, int S, bool WIRE, typename PtrFn>
__device__ __forceinline__ void fold_ring_quads_any(PtrFn ptr, int K, int j, int64_t g0, int64_t gu,
                                                    float acc[S][4]) {
    constexpr int SG = kAnySlices<TIn, S>;
    constexpr int B = kAnyBatch;
    constexpr uintptr_t QB = 4 * sizeof(TIn);
    const int Kr = KS > 0 ? KS : K;
#pragma unroll
    for (int k0 = 0; k0 < S; k0 += SG) {
        for (int h0 = 0; h0 < Kr; h0 += B) {
            Quad<TIn> lo[SG][B], hi[SG][B];
            uint32_t sig[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (h0 + b < Kr) {
                    const char* p = static_cast<const char*>(ptr(wrap(j + h0 + b, Kr)));
                    sig[b] = (uint32_t)(((uintptr_t)p + (uintptr_t)gu * sizeof(TIn)) & (QB - 1));
                    const char* pl = p - sig[b];  // rank base moved back onto the grid
#pragma unroll
                    for (int k = 0; k < SG; ++k) {
                        const int64_t off = (g0 + 256 * (k0 + k)) * (int64_t)sizeof(TIn);
                        lo[k][b] = load_quad<TIn, NT>(reinterpret_cast<const TIn*>(pl + off));
                        hi[k][b] = Quad<TIn>{};
                        if (sig[b]) hi[k][b] = load_quad<TIn, NT>(reinterpret_cast<const TIn*>(pl + QB + off));
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (h0 + b < Kr) {
#pragma unroll
                    for (int k = 0; k < SG; ++k) {
                        const Quad<TIn> q = join_quad(lo[k][b], hi[k][b], sig[b]);
                        if (h0 + b == 0) {
                            widen4(q, acc[k0 + k]);
                        } else {
                            float f[4];
                            widen4(q, f);
                            hop4<WIRE>(acc[k0 + k], f);
                        }
                    }
                }
            }
        }
    }
}

// Free order over ranks in any quad phases: the association of
// fold_free_quads (ranks 0..K-1 in batches of eight, each batch summed as a
// balanced pairwise tree, batches added in sequence), with every rank's quad
// read as an aligned pair. The ranks' order does not depend on the chunk, so
// the phases stay uniform whenever gu and the pointers are.
template <typename TIn, int KS, bool NT, int S, typename PtrFn>
__device__ __forceinline__ void fold_free_quads_any(PtrFn ptr, int K, int64_t g0, int64_t gu, float acc[S][4]) {
    constexpr int SG = kAnySlices<TIn, S>;
    constexpr int B = 8;
    constexpr uintptr_t QB = 4 * sizeof(TIn);
    const int Kr = KS > 0 ? KS : K;
#pragma unroll
    for (int k0 = 0; k0 < S; k0 += SG) {
        for (int h0 = 0; h0 < Kr; h0 += B) {
            Quad<TIn> lo[SG][B], hi[SG][B];
            uint32_t sig[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (h0 + b < Kr) {
                    const char* p = static_cast<const char*>(ptr(h0 + b));
                    sig[b] = (uint32_t)(((uintptr_t)p + (uintptr_t)gu * sizeof(TIn)) & (QB - 1));
                    const char* pl = p - sig[b];
#pragma unroll
                    for (int k = 0; k < SG; ++k) {
                        const int64_t off = (g0 + 256 * (k0 + k)) * (int64_t)sizeof(TIn);
                        lo[k][b] = load_quad<TIn, NT>(reinterpret_cast<const TIn*>(pl + off));
                        hi[k][b] = Quad<TIn>{};
                        if (sig[b]) hi[k][b] = load_quad<TIn, NT>(reinterpret_cast<const TIn*>(pl + QB + off));
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < SG; ++k) {
                // as in fold_free_quads: the first level straight from the
                // loaded pairs, the levels above over the pairs' sums
                float f[B / 2][4];
#pragma unroll
                for (int q = 0; q < B / 2; ++q) {
                    if (h0 + 2 * q < Kr) {
                        widen4(join_quad(lo[k][2 * q], hi[k][2 * q], sig[2 * q]), f[q]);
                        if (h0 + 2 * q + 1 < Kr) {
                            float t[4];
                            widen4(join_quad(lo[k][2 * q + 1], hi[k][2 * q + 1], sig[2 * q + 1]), t);
#pragma unroll
                            for (int e = 0; e < 4; ++e) f[q][e] = __fadd_rn(f[q][e], t[e]);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[q][e] = 0.0f;
                    }
                }
#pragma unroll
                for (int st = 1; st < B / 2; st *= 2)
#pragma unroll
                    for (int q = 0; q + st < B / 2; q += 2 * st)
                        if (h0 + 2 * (q + st) < Kr)
#pragma unroll
                            for (int e = 0; e < 4; ++e) f[q][e] = __fadd_rn(f[q][e], f[q + st][e]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[k0 + k][e] = (h0 == 0) ? f[0][e] : __fadd_rn(acc[k0 + k][e], f[0][e]);
            }
        }
    }
}

}  // namespace zr
