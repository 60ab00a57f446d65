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

// tk_mix: the reduce-scatter's memory access pattern with no arithmetic, the
// practical ceiling of a stream with its read:write mix. K = 8 bf16 input
// streams of n = 8 * C elements and 8 fp32 output streams of C elements; C is a
// multiple of 4096, so every tile is whole, starts on a 128-byte line of every
// input and writes an aligned block of its output. Tiles are numbered as the
// reduce-scatter numbers them: by pairs of chunks, consecutive blocks
// alternating between the pair's two chunks, one block per tile. A tile is
// 4 waves x S slices x 256 elements (S = 1: 4 KiB of output, S = 4: 16 KiB,
// the reduce-scatter's two tile shapes); lane l owns elements 4l..4l+3 of each
// slice and loads them from every input with one 8-byte non-temporal load
// (all 8 S loads issued before the first use), then writes one 16-byte
// non-temporal store per slice to out_j. The stored words are the XOR of the
// loaded ones, so no load can be removed and no floating-point add is made.
//   mode 0: loads and stores (the reduce-scatter's 16 B read : 4 B written)
//   mode 1: loads only (one 16-byte word per tile, written only when the
//           XOR of the tile's data hits a fixed value, keeps the loads live)
//   mode 2: stores only (the same output blocks, no loads)
//   mode 3: mode 0 plus a 16-byte non-temporal load of each output word before
//           its store, folded into the stored value (the accumulating
//           reduce-scatter's 20 B read : 4 B written)
typedef unsigned int tk_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int tk_u32x4 __attribute__((ext_vector_type(4)));

struct TkMixArgs {
    const tk_u32x2* in[8];  // 8 inputs, n bf16 each (4 per 8-byte word)
    tk_u32x4* out[8];       // 8 outputs, C fp32 each (4 per 16-byte word)
    tk_u32x4* sink;         // mode 1: one word per tile
    long long C;            // chunk size (elements), a multiple of 4096
    long long tpc;          // tiles per chunk, C / (1024 S)
    int mode;
};

template <int S>
__global__ void __launch_bounds__(256) tk_mix_kernel(const TkMixArgs a) {
    const long long i = blockIdx.x;
    const long long per_pair = 2 * a.tpc;
    const int q = (int)(i / per_pair);
    const long long w = i - q * per_pair;
    const int j = 2 * q + (int)(w & 1);
    const long long t = w >> 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long o0 = t * (1024 * S) + wave * (256 * S) + lane * 4;  // element offset in the chunk
    const long long g0 = (long long)j * a.C + o0;                        // element index in the inputs
    tk_u32x4* out = a.out[j];
    if (a.mode == 2) {
        const tk_u32x4 v = {(unsigned)o0, (unsigned)j, 0u, 0u};
#pragma unroll
        for (int k = 0; k < S; ++k) __builtin_nontemporal_store(v, out + (o0 + 256 * k) / 4);
        return;
    }
    tk_u32x2 v[S][8];
#pragma unroll
    for (int k = 0; k < S; ++k)
#pragma unroll
        for (int h = 0; h < 8; ++h) v[k][h] = __builtin_nontemporal_load(a.in[h] + (g0 + 256 * k) / 4);
    tk_u32x4 x[S];
#pragma unroll
    for (int k = 0; k < S; ++k) {
        tk_u32x2 y = v[k][0];
#pragma unroll
        for (int h = 1; h < 8; ++h) y ^= v[k][h];
        x[k] = tk_u32x4{y.x, y.y, y.x ^ y.y, y.y + 1u};
    }
    if (a.mode == 0) {
#pragma unroll
        for (int k = 0; k < S; ++k) __builtin_nontemporal_store(x[k], out + (o0 + 256 * k) / 4);
        return;
    }
    if (a.mode == 3) {
        tk_u32x4 old[S];
#pragma unroll
        for (int k = 0; k < S; ++k) old[k] = __builtin_nontemporal_load(out + (o0 + 256 * k) / 4);
#pragma unroll
        for (int k = 0; k < S; ++k) __builtin_nontemporal_store(x[k] ^ old[k], out + (o0 + 256 * k) / 4);
        return;
    }
    tk_u32x4 z = x[0];
#pragma unroll
    for (int k = 1; k < S; ++k) z ^= x[k];
    if (z.x == 0x9E3779B9u && z.y == 0x7F4A7C15u) a.sink[i] = z;
}

extern "C" int tk_mix(const void* const* in, void* const* out, void* sink, long long C, int mode,
                      int slices, void* stream) {
    if (!in || !out || C <= 0 || (C % 4096) != 0 || mode < 0 || mode > 3) return 1;
    if (slices != 1 && slices != 4) return 1;
    if (mode == 1 && !sink) return 1;
    TkMixArgs a;
    for (int r = 0; r < 8; ++r) {
        if (!in[r] || !out[r]) return 1;
        a.in[r] = (const tk_u32x2*)in[r];
        a.out[r] = (tk_u32x4*)out[r];
    }
    a.sink = (tk_u32x4*)sink;
    a.C = C;
    a.tpc = C / (1024LL * slices);
    a.mode = mode;
    const long long blocks = 8 * a.tpc;  // mode 1's sink holds one 16-byte word per block
    if (blocks > (1LL << 30)) return 1;
    if (slices == 1)
        hipLaunchKernelGGL(tk_mix_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(tk_mix_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
