// act_quant.hip -- RMSNorm + per-token absmax int8 quantisation (gfx950).
//
// [huggingface/transformers PR #38087 "Add optional RMSNorm support to BitNet
// quantization (config + layers)", "What does this PR do?": the BitNet
// RMSNorm (eps default 1e-6) runs on the activations before quantisation.]
// [eejd/cpp-bitnet PR #7, NEON-kernel commit: the activations enter the
// ternary dot product as int8 together with their sum.]
//
// Short rows (K <= 1024): one wave per row (wave_act_quant_row, no LDS, no
// barrier).  Longer rows: one 256-thread block per row (block_act_quant_row)
// holding the whole row of x and gamma in registers -- CH float4 of each per
// thread, CH picked from K -- so every row is read with a single round trip
// of fully issued loads.  HBM traffic per row: 4K (x) + 4K (gamma, L2-
// resident after the first rows) + K (q) + 8 bytes.
#include "common.hpp"

namespace bl {
namespace {

struct GlobalRowSink {
    int8_t *q;  // row base
    float *inv;
    int32_t *qsum;
    __device__ void store_q(int k, uint32_t v) { *reinterpret_cast<uint32_t *>(q + k) = v; }
    __device__ void store_row(float iv, int qs) {
        *inv = iv;
        *qsum = qs;
    }
};

__global__ __launch_bounds__(64) void act_quant_wave_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    wave_act_quant_row<1>(x + (size_t)m * K, gamma, eps, K, sink);
}

template <int CH>
__global__ __launch_bounds__(256) void act_quant_block_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    block_act_quant_row<CH, false>(x + (size_t)m * K, gamma, eps, K, red, sink, [] {});
}

__global__ __launch_bounds__(256) void act_quant_long_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    block_act_quant_row<8, true>(x + (size_t)m * K, gamma, eps, K, red, sink, [] {});
}

template <int CH>
hipError_t launch_block(const float *x, const float *gamma, float eps, int64_t M, int64_t K,
                        int8_t *q, float *inv, int32_t *qsum, hipStream_t s) {
    hipLaunchKernelGGL(act_quant_block_kernel<CH>, dim3((unsigned)M), dim3(256), 0, s, x, gamma,
                       eps, (int)K, q, inv, qsum);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const float *x, const float *gamma, float eps,
                            int64_t M, int64_t K, int8_t *q, float *inv,
                            int32_t *qsum, hipStream_t s) {
    if (K <= 1024) {
        hipLaunchKernelGGL(act_quant_wave_kernel, dim3((unsigned)M), dim3(64), 0, s, x, gamma,
                           eps, (int)K, q, inv, qsum);
        return hipGetLastError();
    }
    if (K <= 4 * 1024) return launch_block<4>(x, gamma, eps, M, K, q, inv, qsum, s);
    if (K <= 8 * 1024) return launch_block<8>(x, gamma, eps, M, K, q, inv, qsum, s);
    if (K <= 16 * 1024) return launch_block<16>(x, gamma, eps, M, K, q, inv, qsum, s);
    if (K <= 32 * 1024) return launch_block<32>(x, gamma, eps, M, K, q, inv, qsum, s);
    // Rows beyond 32768: streamed in three passes.
    hipLaunchKernelGGL((act_quant_long_kernel), dim3((unsigned)M), dim3(256), 0, s, x, gamma, eps,
                       (int)K, q, inv, qsum);
    return hipGetLastError();
}

}  // namespace bl
