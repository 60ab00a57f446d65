// IPG bucket flatten: fragmented gradients copied into one flat bucket per
// rank at running offsets, then the bucket's tail zero-filled up to the
// padded size ("DeepSpeed ZeRO-3 源码解析", 3.2 and 5.1: each grad lives at
// offset n_0 + ... + n_{p-1} of the flat buffer; 3.1: one large contiguous
// message instead of one per parameter).
//
// A launch carries up to 96 copy jobs in its kernel arguments (no device
// descriptor table, no staging copy). blockIdx.y = job, blockIdx.x strides
// over 4 KiB tiles of the job; a lane moves 16 bytes. When source and
// destination are both 16-byte aligned the lane copies with one 16-byte load
// and store; otherwise (the usual case inside a bucket, since offsets are
// prefix sums of arbitrary sizes) it copies its 16 destination bytes element
// by element. A job with no source writes zeros.
#include "zr_device.hpp"
#include "zr_internal.hpp"

namespace zr {
namespace {

constexpr int kFlatTileBytes = kThreads * 16;

struct FlatArgs {
    CopyJob job[kFlatJobsPerLaunch];
    int es;  // element bytes, 2 or 4
};

template <typename T>
__device__ __forceinline__ void copy_elems(const T* src, T* dst, int n) {
    if (src) {
        for (int e = 0; e < n; ++e) dst[e] = src[e];
    } else {
        for (int e = 0; e < n; ++e) dst[e] = T(0);
    }
}

template <typename T>
__global__ void __launch_bounds__(kThreads) flatten_kernel(const FlatArgs a) {
    const CopyJob jb = a.job[blockIdx.y];
    const int64_t bytes = jb.n * (int64_t)sizeof(T);
    const int64_t tiles = (bytes + kFlatTileBytes - 1) / kFlatTileBytes;
    const bool vec = ((((uintptr_t)jb.dst) & 15) == 0) &&
                     (jb.src == nullptr || (((uintptr_t)jb.src) & 15) == 0);
    constexpr int per = 16 / sizeof(T);  // elements per lane
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t e0 = (t * kFlatTileBytes + (int64_t)threadIdx.x * 16) / (int64_t)sizeof(T);
        if (e0 >= jb.n) continue;
        T* d = static_cast<T*>(jb.dst) + e0;
        const T* s = jb.src ? static_cast<const T*>(jb.src) + e0 : nullptr;
        if (vec && e0 + per <= jb.n) {
            u32x4 v = s ? *reinterpret_cast<const u32x4*>(s) : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(d) = v;
        } else {
            const int n = (int)((jb.n - e0) < per ? (jb.n - e0) : per);
            copy_elems<T>(s, d, n);
        }
    }
}

}  // namespace

hipError_t launch_flatten(const CopyJob* jobs, int n_jobs, int elem_bytes, hipStream_t stream) {
    if (n_jobs <= 0) return hipSuccess;
    FlatArgs a;
    a.es = elem_bytes;
    int64_t max_tiles = 1;
    for (int i = 0; i < n_jobs; ++i) {
        a.job[i] = jobs[i];
        const int64_t t = (jobs[i].n * elem_bytes + kFlatTileBytes - 1) / kFlatTileBytes;
        if (t > max_tiles) max_tiles = t;
    }
    int64_t want = (int64_t)device_cu_count() * 8 / n_jobs;
    if (want < 1) want = 1;
    const int gx = (int)(want < max_tiles ? want : max_tiles);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(flatten_kernel<uint16_t>, dim3(gx, n_jobs), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(flatten_kernel<uint32_t>, dim3(gx, n_jobs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace zr
