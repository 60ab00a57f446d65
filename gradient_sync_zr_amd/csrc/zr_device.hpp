// Device helpers shared by the HIP kernels: the bf16 codec, streaming loads
// and stores, the 16-byte realignment of copies between grids, quad loads and
// stores, the tile searches and the average.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zr {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // threads per block (4 waves of 64)

// bf16 <-> fp32. bf16 is the upper half of an IEEE binary32 word, so widening
// appends 16 zero bits (exact). Narrowing rounds to nearest, ties to even;
// a NaN keeps its sign and top payload bits and is forced quiet.
__device__ __forceinline__ float bf16_widen(uint32_t h16) { return __uint_as_float(h16 << 16); }

__device__ __forceinline__ uint32_t bf16_round(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT, typename V>
__device__ __forceinline__ void st(V* p, V v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// 16 bytes starting `sig` bytes into the 32 bytes lo:hi (sig in 1..15, a
// multiple of the element size): each output dword joins two neighbouring
// input dwords with one byte-align instruction.
__device__ __forceinline__ u32x4 shift16(const u32x4& lo, const u32x4& hi, uint32_t sig) {
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const uint32_t b = sig & 3;
    u32x4 r;
#define ZR_SHIFT16(q)                                                   \
    r = u32x4{__builtin_amdgcn_alignbyte(w[(q) + 1], w[(q)], b),          \
              __builtin_amdgcn_alignbyte(w[(q) + 2], w[(q) + 1], b),      \
              __builtin_amdgcn_alignbyte(w[(q) + 3], w[(q) + 2], b),      \
              __builtin_amdgcn_alignbyte(w[(q) + 4], w[(q) + 3], b)}
    switch (sig >> 2) {  // uniform in every caller: the phase of a whole copy
        case 0: ZR_SHIFT16(0); break;
        case 1: ZR_SHIFT16(1); break;
        case 2: ZR_SHIFT16(2); break;
        default: ZR_SHIFT16(3); break;
    }
#undef ZR_SHIFT16
    return r;
}

// Scalar element access for the unaligned / ragged paths.
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_widen(*p); }
__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = (uint16_t)bf16_round(v); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }

// The slot holding item t of a flat item space cut into n slots, where
// start[0..n] is nondecreasing, start[0] = 0 and start[n] > t; the search
// begins at slot m (a lower bound). The wave's lanes read 64 starts at once
// and count those <= t with a ballot: the slot is the last of them (empty
// slots, whose start repeats the next one's, are passed over). t and m are
// uniform across the wave; one round unless t lies 64 or more slots ahead.
__device__ __forceinline__ int find_slot(const int32_t* start, int n, int m, int t) {
    const int lane = threadIdx.x & 63;
    while (true) {
        const int idx = m + lane;
        const bool le = idx <= n && start[idx <= n ? idx : n] <= t;
        const int c = __popcll(__ballot(le));
        if (c < 64) return m + c - 1;
        m += 64;
    }
}

// A pointer into a descriptor table staged in device memory, in the constant
// address space: the table is read-only while a kernel runs, so loads at a
// block-uniform index become scalar loads. Tables pass their device address
// as an integer in the kernel arguments.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ cptr<T> table_at(uint64_t addr) {
    return reinterpret_cast<cptr<T>>(addr);
}

// The slot holding item t of a flat item space cut into n slots, where
// start[0..n] (a staged table) is nondecreasing, start[0] = 0 <= t < start[n]:
// the last s with start[s] <= t. The wave narrows [lo, hi) 64 candidates at
// a time (one load per lane, a ballot counts those <= t), so any n is found in
// ceil(log64 n) rounds. t is uniform across the wave.
__device__ __forceinline__ int64_t find_slot64(cptr<int64_t> start, int64_t n, int64_t t) {
    const int lane = threadIdx.x & 63;
    int64_t lo = 0, hi = n;  // start[lo] <= t < start[hi]
    while (hi - lo > 1) {
        const int64_t step = (hi - lo + 63) / 64;
        const int64_t idx = lo + (int64_t)lane * step;
        const bool le = idx < hi && start[idx] <= t;  // true on a prefix of the lanes
        const int c = __popcll(__ballot(le));        // >= 1: lane 0 reads start[lo]
        const int64_t nhi = lo + (int64_t)c * step;
        lo += (int64_t)(c - 1) * step;
        hi = nhi < hi ? nhi : hi;
    }
    return lo;
}

// Average: AVG 0 = none, 1 = multiply by the exact reciprocal (K a power of
// two, identical to dividing), 2 = IEEE correctly rounded divide by K.
template <int AVG>
__device__ __forceinline__ float average(float s, float inv_k, float kf) {
    if constexpr (AVG == 1) return __fmul_rn(s, inv_k);
    if constexpr (AVG == 2) return __fdiv_rn(s, kf);
    return s;
}

}  // namespace zr

// ---------------------------------------------------------------- quads
// A quad is 4 consecutive elements: 8 bytes of bf16 or 16 bytes of fp32.
// Kernels that lay lanes out on quads make every load and store instruction
// of a wave cover one contiguous span (64 lanes x 4 elements), so stores
// write whole cache lines per instruction.
namespace zr {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Quad;
template <>
struct Quad<uint16_t> {
    u32x2 v;
};
template <>
struct Quad<float> {
    f32x4 v;
};

template <typename T, bool NT>
__device__ __forceinline__ Quad<T> load_quad(const T* p) {
    if constexpr (sizeof(T) == 2)
        return {ld<NT>(reinterpret_cast<const u32x2*>(p))};
    else
        return {ld<NT>(reinterpret_cast<const f32x4*>(p))};
}

__device__ __forceinline__ void widen4(const Quad<uint16_t>& q, float f[4]) {
    f[0] = __uint_as_float(q.v.x << 16);
    f[1] = __uint_as_float(q.v.x & 0xFFFF0000u);
    f[2] = __uint_as_float(q.v.y << 16);
    f[3] = __uint_as_float(q.v.y & 0xFFFF0000u);
}
__device__ __forceinline__ void widen4(const Quad<float>& q, float f[4]) {
    f[0] = q.v.x; f[1] = q.v.y; f[2] = q.v.z; f[3] = q.v.w;
}

template <typename T>
__device__ __forceinline__ void accumulate4(float acc[4], const Quad<T>& q) {
    float f[4];
    widen4(q, f);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __fadd_rn(acc[e], f[e]);
}

template <typename T>
__device__ __forceinline__ Quad<T> pack4(const float f[4]);
template <>
__device__ __forceinline__ Quad<uint16_t> pack4<uint16_t>(const float f[4]) {
    Quad<uint16_t> q;
    q.v.x = bf16_round(f[0]) | (bf16_round(f[1]) << 16);
    q.v.y = bf16_round(f[2]) | (bf16_round(f[3]) << 16);
    return q;
}
template <>
__device__ __forceinline__ Quad<float> pack4<float>(const float f[4]) {
    return {f32x4{f[0], f[1], f[2], f[3]}};
}

template <typename T, bool NT>
__device__ __forceinline__ void store_quad(T* p, const Quad<T>& q) {
    if constexpr (sizeof(T) == 2)
        st<NT>(reinterpret_cast<u32x2*>(p), q.v);
    else
        st<NT>(reinterpret_cast<f32x4*>(p), q.v);
}

}  // namespace zr
