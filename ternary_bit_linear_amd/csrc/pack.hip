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

// Word s (0..7) of block b of row n holds, in byte i and field g, the code
// of weight 128b + 32g + 4s + i.  A thread builds one word per loop trip:
// the eight threads of a block read, per field g, the 32 consecutive
// weights 128b + 32g + [0, 32) as eight float4, so every load instruction
// of a wave reads whole 128-byte lines (8 blocks x 128 bytes) and the wave
// writes 256 consecutive output bytes.  The grid is capped and strides over
// the words, so the minimum and maximum stay in registers for many words
// and each workgroup touches the trailer words at most once: one hot
// address read by every wave of a one-word-per-thread grid serialises at
// the memory channel that owns it.  I is 32-bit whenever the word count
// fits, which keeps the row division cheap.
template <typename I>
__global__ __launch_bounds__(256) void pack_scan_kernel(const float *__restrict__ w, I words,
                                                         I words_per_row, I K,
                                                         uint8_t *__restrict__ packed,
                                                         uint32_t *__restrict__ stats) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    uint32_t mn = 0xffffffffu, mx = 0u;
    const I stride = (I)gridDim.x * blockDim.x;
    for (I u = (I)blockIdx.x * blockDim.x + threadIdx.x; u < words; u += stride) {
        const I n = u / words_per_row;
        const I r = u - n * words_per_row;
        const float *src = w + (int64_t)n * K + (int64_t)(r >> 3) * kBlockWeights + 4 * (r & 7);
        // W is read once: non-temporal loads keep it from displacing
        // cached lines (measured about 10% faster than plain loads).
        f4v v[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            v[g] = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(src + 32 * g));
        uint32_t word = 0u;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int sh = 6 - 2 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = v[g][i];
                const uint32_t code = e > 0.0f ? 2u : (e < 0.0f ? 0u : 1u);
                word |= code << (8 * i + sh);
                const uint32_t bits = __float_as_uint(e) & 0x7fffffffu;
                if (bits != 0u) {
                    mn = min(mn, bits);
                    mx = max(mx, bits);
                }
            }
        }
        reinterpret_cast<uint32_t *>(packed)[u] = word;
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    __shared__ uint32_t part[2][4];
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        part[0][wv] = mn;
        part[1][wv] = mx;
    }
    __syncthreads();
    // Fold into the trailer words only where this workgroup can improve
    // them.  The words only ever move towards their final values, so a
    // stale read can at worst cause a needless atomic, never skip a needed
    // one.
    if (threadIdx.x == 0) {
        const int nw = (blockDim.x + 63) >> 6;
        for (int i = 1; i < nw; ++i) {
            mn = min(mn, part[0][i]);
            mx = max(mx, part[1][i]);
        }
        const uint32_t cur_mn = __hip_atomic_load(stats + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t cur_mx = __hip_atomic_load(stats + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (mn < cur_mn) atomicMin(stats + 0, mn);
        if (mx > cur_mx) atomicMax(stats + 1, mx);
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

// One thread per 4-byte packed word (16 weights w = (code - 1) * scale):
// the mirror of pack_scan_kernel's mapping, so the stores of a wave fill
// whole 128-byte lines (64 for the half types).  OT: the output type; the
// fp32 value (code - 1) * scale is rounded to it to nearest even.
template <typename OT>
__device__ __forceinline__ void store4(OT *dst, float a, float b, float c, float d) {
    if constexpr (std::is_same<OT, float>::value) {
        *reinterpret_cast<float4 *>(dst) = make_float4(a, b, c, d);
    } else {
        const uint32_t lo = (uint32_t)to_half_bits<OT>(a) | ((uint32_t)to_half_bits<OT>(b) << 16);
        const uint32_t hi = (uint32_t)to_half_bits<OT>(c) | ((uint32_t)to_half_bits<OT>(d) << 16);
        *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
    }
}

template <typename OT = float>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed,
                                                      int64_t words, int64_t words_per_row,
                                                      int64_t K, const float *__restrict__ scale_p,
                                                      OT *__restrict__ w) {
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= words) return;
    const float s = *scale_p;
    const uint32_t d = reinterpret_cast<const uint32_t *>(packed)[u];
    const int64_t n = u / words_per_row;
    const int64_t r = u - n * words_per_row;
    OT *dst = w + n * K + (r >> 3) * kBlockWeights + 4 * (r & 7);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int sh = 6 - 2 * g;
        store4(dst + 32 * g, (float)((int)((d >> sh) & 3u) - 1) * s,
               (float)((int)((d >> (sh + 8)) & 3u) - 1) * s,
               (float)((int)((d >> (sh + 16)) & 3u) - 1) * s,
               (float)((int)((d >> (sh + 24)) & 3u) - 1) * s);
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
    const int64_t wpr = K / 16;
    const int64_t words = N * wpr;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    // Four 256-thread workgroups per CU: measured as fast as more.
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((words + 255) / 256, 4 * (int64_t)cus));
    uint32_t *stats = reinterpret_cast<uint32_t *>(packed + N * (K / 4));
    if (words + 256 * blocks < (int64_t)UINT32_MAX)
        hipLaunchKernelGGL(pack_scan_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                           w, (uint32_t)words, (uint32_t)wpr, (uint32_t)K, packed, stats);
    else
        hipLaunchKernelGGL(pack_scan_kernel<int64_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                           w, words, wpr, K, packed, stats);
    return hipGetLastError();
}

hipError_t launch_pack_finalize(uint8_t *trailer, float scale, hipStream_t s) {
    hipLaunchKernelGGL(pack_finalize_kernel, dim3(1), dim3(64), 0, s,
                       reinterpret_cast<uint32_t *>(trailer), scale);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t N, int64_t K, float *w,
                         hipStream_t s) {
    return launch_dequant(packed, N, K, w, kIoF32, s);
}

hipError_t launch_dequant(const uint8_t *packed, int64_t N, int64_t K, void *w, int wtype,
                          hipStream_t s) {
    const int64_t wpr = K / 16;
    const int64_t words = N * wpr;
    const int64_t blocks = (words + 255) / 256;
    const float *scale_p = reinterpret_cast<const float *>(packed + N * (K / 4));
    const dim3 grid((unsigned)blocks), block(256);
    switch (wtype) {
        case kIoF32:
            hipLaunchKernelGGL(unpack_kernel<float>, grid, block, 0, s, packed, words, wpr, K,
                               scale_p, static_cast<float *>(w));
            break;
        case kIoBf16:
            hipLaunchKernelGGL(unpack_kernel<bf16_t>, grid, block, 0, s, packed, words, wpr, K,
                               scale_p, static_cast<bf16_t *>(w));
            break;
        case kIoF16:
            hipLaunchKernelGGL(unpack_kernel<_Float16>, grid, block, 0, s, packed, words, wpr, K,
                               scale_p, static_cast<_Float16 *>(w));
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bl
