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
