// Seeded synthetic inputs, device side: the same counter-based generator as
// synth_host.c (SplitMix64 evaluated at a counter, Irwin-Hall normals with
// twelve 16-bit terms, fp32 scale, round-to-nearest-even to bf16), written
// for the GPU so that large inputs never cross PCIe. The two sides must agree
// bit for bit; tests compare them on sampled indices.
//
// Input tooling only: nothing here is part of the gradient reduction.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;
constexpr uint64_t kStreamMul = 0xD1B54A32D192ED03ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__host__ uint64_t mix64_host(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word_at(uint64_t key, uint64_t n) {
    return mix64(key + (n + 1) * kGamma);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float normal_value(uint64_t key, uint64_t e, float sigma,
                                              uint32_t thr, float mag) {
    int32_t s = 0;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        uint64_t x = word_at(key, 4 * e + (uint64_t)w);
        s += (int32_t)(x & 0xFFFF) + (int32_t)((x >> 16) & 0xFFFF) +
             (int32_t)((x >> 32) & 0xFFFF) + (int32_t)((x >> 48) & 0xFFFF);
    }
    float z = __fmul_rn((float)(s - 6 * 65536), 1.0f / 65536.0f);
    float v = __fmul_rn(z, sigma);
    if (thr != 0) {
        uint64_t x = word_at(key, 4 * e + 3);
        if ((uint32_t)(x >> 32) < thr) v = (x & 1u) ? -mag : mag;
    }
    return v;
}

__device__ __forceinline__ int32_t uniform_int(uint64_t key, uint64_t e, int32_t lo, int32_t hi) {
    uint64_t m = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
    uint64_t x = word_at(key, 4 * e);
    return (int32_t)((int64_t)lo + (int64_t)(((x >> 32) * m) >> 32));
}

enum Kind { kNormalBf16 = 0, kIntF32 = 1, kIntBf16 = 2 };

// Each thread writes groups of 8 consecutive elements; a group that is whole
// and 16-byte aligned goes out as one 16-byte store, anything else element by
// element. Grid-stride over groups; every index is checked against `count`.
template <int KIND>
__global__ void __launch_bounds__(256) fill_kernel(uint64_t key, uint64_t start, uint64_t count,
                                                   float sigma, uint32_t thr, float mag,
                                                   int32_t lo, int32_t hi, void* dst) {
    const uint64_t groups = (count + 7) / 8;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t gidx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; gidx < groups;
         gidx += stride) {
        const uint64_t i0 = gidx * 8;
        if (KIND == kIntF32) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                v[k] = (float)uniform_int(key, start + i0 + k, lo, hi);
            float* d = (float*)dst + i0;
            if (i0 + 8 <= count && (((uintptr_t)d) & 15) == 0) {
                reinterpret_cast<float4*>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
                reinterpret_cast<float4*>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else {
                for (int k = 0; k < 8 && i0 + k < count; ++k) d[k] = v[k];
            }
        } else {
            uint16_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float f = (KIND == kNormalBf16)
                              ? normal_value(key, start + i0 + k, sigma, thr, mag)
                              : (float)uniform_int(key, start + i0 + k, lo, hi);
                v[k] = to_bf16(f);
            }
            uint16_t* d = (uint16_t*)dst + i0;
            if (i0 + 8 <= count && (((uintptr_t)d) & 15) == 0) {
                uint4 p;
                p.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
                p.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
                p.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
                p.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
                *reinterpret_cast<uint4*>(d) = p;
            } else {
                for (int k = 0; k < 8 && i0 + k < count; ++k) d[k] = v[k];
            }
        }
    }
}

int launch(int kind, uint64_t seed, uint64_t stream_id, uint64_t start, uint64_t count,
           float sigma, uint32_t thr, float mag, int32_t lo, int32_t hi, void* dst,
           void* stream) {
    if (count == 0) return 0;
    if (dst == nullptr) return 1;
    const uint64_t key = mix64_host(seed ^ (stream_id * kStreamMul));
    const uint64_t groups = (count + 7) / 8;
    uint64_t blocks = (groups + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipStream_t s = (hipStream_t)stream;
    switch (kind) {
        case kNormalBf16:
            hipLaunchKernelGGL(fill_kernel<kNormalBf16>, dim3((unsigned)blocks), dim3(256), 0, s,
                               key, start, count, sigma, thr, mag, lo, hi, dst);
            break;
        case kIntF32:
            hipLaunchKernelGGL(fill_kernel<kIntF32>, dim3((unsigned)blocks), dim3(256), 0, s, key,
                               start, count, sigma, thr, mag, lo, hi, dst);
            break;
        case kIntBf16:
            hipLaunchKernelGGL(fill_kernel<kIntBf16>, dim3((unsigned)blocks), dim3(256), 0, s,
                               key, start, count, sigma, thr, mag, lo, hi, dst);
            break;
        default:
            return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" {

// All return 0 on success, 1 on a bad argument, 2 on a launch error.
// `dst` is device memory holding `count` elements; `stream` is a hipStream_t.
int synth_dev_normal_bf16(uint64_t seed, uint64_t stream_id, uint64_t start, uint64_t count,
                          float sigma, uint32_t thr, float mag, void* dst, void* stream) {
    return launch(kNormalBf16, seed, stream_id, start, count, sigma, thr, mag, 0, 0, dst, stream);
}

int synth_dev_uniform_int_f32(uint64_t seed, uint64_t stream_id, uint64_t start, uint64_t count,
                              int32_t lo, int32_t hi, void* dst, void* stream) {
    if (hi < lo) return 1;
    return launch(kIntF32, seed, stream_id, start, count, 0.f, 0, 0.f, lo, hi, dst, stream);
}

int synth_dev_uniform_int_bf16(uint64_t seed, uint64_t stream_id, uint64_t start, uint64_t count,
                               int32_t lo, int32_t hi, void* dst, void* stream) {
    if (hi < lo) return 1;
    return launch(kIntBf16, seed, stream_id, start, count, 0.f, 0, 0.f, lo, hi, dst, stream);
}

}  // extern "C"
