// Test helper kernels (test infrastructure only, not part of libzr).
//
// tk_delay: one wave that spins on the constant-rate wall clock for a bounded
// number of ticks, to hold a stream busy while a test checks what other
// streams may or may not do meanwhile. The loop ends after `ticks` wall-clock
// ticks or after `max_iters` iterations, whichever comes first, so it always
// exits.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ void tk_delay_kernel(long long ticks, long long max_iters, unsigned int* done_flag) {
    const long long t0 = wall_clock64();
    long long it = 0;
    while (wall_clock64() - t0 < ticks && it < max_iters) {
        __builtin_amdgcn_s_sleep(16);
        ++it;
    }
    if (threadIdx.x == 0 && done_flag) *done_flag = 1u;
}

extern "C" int tk_delay(long long ticks, long long max_iters, void* done_flag, void* stream) {
    if (ticks < 0 || max_iters < 0) return 1;
    hipLaunchKernelGGL(tk_delay_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ticks, max_iters,
                       (unsigned int*)done_flag);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Rate (kHz) of the wall clock that wall_clock64() reads, for converting a
// wanted delay into ticks.
extern "C" int tk_clock_khz(int* khz) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 2;
    return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? 0 : 2;
}

// tk_copy: a plain streaming copy of `bytes` bytes (a multiple of 16), each
// lane moving 16 bytes per iteration of a grid-stride loop. Used to calibrate
// the hardware byte counters (a copy reads and writes exactly `bytes`) and as
// the practical HBM ceiling a bandwidth-bound kernel can be compared with.
__global__ void __launch_bounds__(256) tk_copy_kernel(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst, long long n16) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

extern "C" int tk_copy(const void* src, void* dst, long long bytes, int blocks, void* stream) {
    if (bytes < 0 || (bytes & 15) || blocks < 1 || !src || !dst) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(tk_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// tk_read: reads `bytes` bytes (a multiple of 16) and writes one 16-byte
// value per block (so the loads cannot be removed): a read-only stream.
__global__ void __launch_bounds__(256) tk_read_kernel(const uint4* __restrict__ src,
                                                      uint4* __restrict__ sink, long long n16) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        uint4 v = src[i];
        acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
    }
    __shared__ uint4 red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int t = 1; t < 256; ++t) {
            acc.x ^= red[t].x; acc.y ^= red[t].y; acc.z ^= red[t].z; acc.w ^= red[t].w;
        }
        sink[blockIdx.x] = acc;
    }
}

extern "C" int tk_read(const void* src, void* sink, long long bytes, int blocks, void* stream) {
    if (bytes < 0 || (bytes & 15) || blocks < 1 || !src || !sink) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(tk_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)sink, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// tk_xcd: every block of a one-block-per-tile launch copies one 4 KiB tile
// (so blocks retire at varying times, as in the library's kernels) and
// records the XCD it ran on, read from the XCC_ID hardware register (bits
// 3:0), in xcd[blockIdx.x]. src and dst hold blocks * 4 KiB.
__global__ void __launch_bounds__(256) tk_xcd_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, int* __restrict__ xcd) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    dst[i] = src[i];
    if (threadIdx.x == 0) xcd[blockIdx.x] = (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15);
}

extern "C" int tk_xcd(const void* src, void* dst, void* xcd, int blocks, void* stream) {
    if (blocks < 1 || !src || !dst || !xcd) return 1;
    hipLaunchKernelGGL(tk_xcd_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)dst, (int*)xcd);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
