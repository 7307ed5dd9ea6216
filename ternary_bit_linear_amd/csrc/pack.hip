// pack.hip -- I2_S packer and unpacker (gfx950).
//
// [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU FFN",
// summary bullet and commit "llama-quantize I2_S emits the canonical
// layout": one call per tensor; the scale is per tensor and stored after the
// packed data; the 28 unused trailer bytes are zero; scale = first non-zero
// |w|, inputs already ternary x scale; rows divisible by 128.]
//
// The packer is one pass over W.  Codes depend only on the sign (the input
// is ternary x scale), so no scale is needed to write them.  While packing,
// each wave reduces the minimum and maximum bit pattern of the non-zero
// |w| it saw (fp32 bit patterns of non-negative numbers order like the
// numbers; NaN patterns sort above +inf) and folds them into the first two
// words of the trailer with atomics; the host reads those 8 bytes back: on
// valid input min == max == the bits of the one non-zero magnitude, which
// is then also the first non-zero |w|.  A final one-wave kernel writes the
// trailer proper.
#include "common.hpp"

namespace bl {
namespace {

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, s, kWave));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, s, kWave));
    return v;
}

// One thread per 16-byte output chunk: bytes [16h, 16h+16) of block b of row
// n hold, in field g, the weights 128b + 32g + 16h + [0, 16).
__global__ __launch_bounds__(256) void pack_scan_kernel(const float *__restrict__ w,
                                                         int64_t chunks, int64_t chunks_per_row,
                                                         int64_t K, uint8_t *__restrict__ packed,
                                                         uint32_t *__restrict__ stats) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t mn = 0xffffffffu, mx = 0u;
    if (c < chunks) {
        const int64_t n = c / chunks_per_row;
        const int64_t cc = c % chunks_per_row;
        const float *src = w + n * K + (cc >> 1) * kBlockWeights + 16 * (cc & 1);
        uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int sh = 6 - 2 * g;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const float4 v = *reinterpret_cast<const float4 *>(src + 32 * g + 4 * t4);
                const float e[4] = {v.x, v.y, v.z, v.w};
                uint32_t word = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t code = e[i] > 0.0f ? 2u : (e[i] < 0.0f ? 0u : 1u);
                    word |= code << (8 * i + sh);
                    const uint32_t bits = __float_as_uint(e[i]) & 0x7fffffffu;
                    if (bits != 0u) {
                        mn = min(mn, bits);
                        mx = max(mx, bits);
                    }
                }
                d[t4] |= word;
            }
        }
        *reinterpret_cast<uint4 *>(packed + 16 * c) = make_uint4(d[0], d[1], d[2], d[3]);
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if ((threadIdx.x & 63) == 0) {
        if (mn != 0xffffffffu) atomicMin(stats + 0, mn);
        if (mx != 0u) atomicMax(stats + 1, mx);
    }
}

__global__ void pack_init_kernel(uint32_t *trailer) {
    const int t = threadIdx.x;
    if (t < 8) trailer[t] = (t == 0) ? 0xffffffffu : 0u;
}

__global__ void pack_finalize_kernel(uint32_t *trailer, float scale) {
    const int t = threadIdx.x;
    if (t < 8) trailer[t] = (t == 0) ? __float_as_uint(scale) : 0u;
}

// One thread per 16-byte chunk: 64 weights w = (code - 1) * scale.
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed,
                                                      int64_t chunks, int64_t chunks_per_row,
                                                      int64_t K, const float *__restrict__ scale_p,
                                                      float *__restrict__ w) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks) return;
    const float s = *scale_p;
    const uint4 p = *reinterpret_cast<const uint4 *>(packed + 16 * c);
    const uint32_t d[4] = {p.x, p.y, p.z, p.w};
    const int64_t n = c / chunks_per_row;
    const int64_t cc = c % chunks_per_row;
    float *dst = w + n * K + (cc >> 1) * kBlockWeights + 16 * (cc & 1);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int sh = 6 - 2 * g;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            float4 v;
            v.x = (float)((int)((d[t4] >> sh) & 3u) - 1) * s;
            v.y = (float)((int)((d[t4] >> (sh + 8)) & 3u) - 1) * s;
            v.z = (float)((int)((d[t4] >> (sh + 16)) & 3u) - 1) * s;
            v.w = (float)((int)((d[t4] >> (sh + 24)) & 3u) - 1) * s;
            *reinterpret_cast<float4 *>(dst + 32 * g + 4 * t4) = v;
        }
    }
}

}  // namespace

hipError_t launch_pack_init(uint8_t *trailer, hipStream_t s) {
    hipLaunchKernelGGL(pack_init_kernel, dim3(1), dim3(64), 0, s,
                       reinterpret_cast<uint32_t *>(trailer));
    return hipGetLastError();
}

hipError_t launch_pack_scan(const float *w, int64_t N, int64_t K, uint8_t *packed,
                            hipStream_t s) {
    const int64_t cpr = K / 64;
    const int64_t chunks = N * cpr;
    const int64_t blocks = (chunks + 255) / 256;
    uint32_t *stats = reinterpret_cast<uint32_t *>(packed + N * (K / 4));
    hipLaunchKernelGGL(pack_scan_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, chunks,
                       cpr, K, packed, stats);
    return hipGetLastError();
}

hipError_t launch_pack_finalize(uint8_t *trailer, float scale, hipStream_t s) {
    hipLaunchKernelGGL(pack_finalize_kernel, dim3(1), dim3(64), 0, s,
                       reinterpret_cast<uint32_t *>(trailer), scale);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t N, int64_t K, float *w,
                         hipStream_t s) {
    const int64_t cpr = K / 64;
    const int64_t chunks = N * cpr;
    const int64_t blocks = (chunks + 255) / 256;
    const float *scale_p = reinterpret_cast<const float *>(packed + N * (K / 4));
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, packed, chunks,
                       cpr, K, scale_p, w);
    return hipGetLastError();
}

}  // namespace bl
