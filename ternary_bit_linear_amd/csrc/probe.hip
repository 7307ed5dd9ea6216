// probe.hip -- calibration probes for the benchmark (gfx950): the rate at
// which one launch can read a buffer from HBM, and the rate of back-to-back
// int8 MFMAs.  They give the attainable ceilings that the BitLinear kernels'
// roofline fractions are read against (the published peaks assume the
// 2.4 GHz boost clock, which the device does not hold under sustained MFMA
// load).  Not part of the BitLinear path.
#include <algorithm>

#include "common.hpp"

namespace bl {
namespace {

typedef int v16i_p __attribute__((ext_vector_type(16)));

// One pass over `bytes` (a multiple of 16): every thread reads CH 16-byte
// chunks, the chunks of a workgroup's pass contiguous per load instruction
// (coalesced 1 KB per wave load), all loads issued before any is used; the
// XOR of what it read goes to sink[blockIdx] so nothing is elided.
template <int CH>
__global__ __launch_bounds__(256) void probe_read_kernel(const uint8_t *__restrict__ src,
                                                         uint64_t bytes,
                                                         uint32_t *__restrict__ sink) {
    const uint64_t base = (uint64_t)blockIdx.x * (256u * 16u * CH);
    const uint64_t left = bytes > base ? bytes - base : 0;
    const auto r = make_rsrc(src + base, (uint32_t)std::min<uint64_t>(left, 256u * 16u * CH));
    v4i v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = buf_load16(r, (uint32_t)(c * 256 + threadIdx.x) * 16u);
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) x ^= (uint32_t)(v[c].x ^ v[c].y ^ v[c].z ^ v[c].w);
    // one word per workgroup: lane 0 of each wave xors into LDS, then one store
    __shared__ uint32_t part[4];
    for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Back-to-back v_mfma_i32_32x32x32_i8 on four independent accumulators per
// wave, `iters` rounds (4 MFMAs each, 65536 int ops per MFMA); operands are
// fixed registers, so nothing but the matrix core is exercised.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int64_t iters, int32_t *__restrict__ sink) {
    const v4i a = {(int)threadIdx.x, 1, 2, 3}, b = {5, (int)blockIdx.x, 7, 9};
    v16i_p c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] ^ c1[e] ^ c2[e] ^ c3[e];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

int64_t probe_read_blocks(uint64_t bytes) { return (int64_t)((bytes + 256 * 16 * 8 - 1) / (256 * 16 * 8)); }

hipError_t launch_probe_read(const uint8_t *src, uint64_t bytes, uint32_t *sink, hipStream_t s) {
    const int64_t blocks = probe_read_blocks(bytes);
    hipLaunchKernelGGL(probe_read_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, s, src, bytes,
                       sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int64_t iters, int64_t blocks, int32_t *sink, hipStream_t s) {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, s, iters, sink);
    return hipGetLastError();
}

}  // namespace bl
