// act_quant.hip -- RMSNorm + per-token absmax int8 quantisation (gfx950).
//
// [huggingface/transformers PR #38087 "Add optional RMSNorm support to BitNet
// quantization (config + layers)", "What does this PR do?": the BitNet
// RMSNorm (eps default 1e-6) runs on the activations before quantisation.]
// [eejd/cpp-bitnet PR #7, NEON-kernel commit: the activations enter the
// ternary dot product as int8 together with their sum.]
//
// One 256-thread block per 4 token rows; each wave computes one row's sum of
// squares in the fixed order of wave_sumsq, then the block quantises the rows
// one by one with coalesced float4 loads of x and gamma.  HBM traffic is
// 4*M*K bytes of x (re-read from L2 twice), 4*K of gamma, M*K of q out.
#include "common.hpp"

namespace bl {
namespace {

struct GlobalSink {
    int8_t *q;
    float *inv;
    int32_t *qsum;
    int64_t K;
    __device__ void store_q(int m, int k, uint32_t v) {
        *reinterpret_cast<uint32_t *>(q + (size_t)m * K + k) = v;
    }
    __device__ void store_row(int m, float iv, int qs) {
        inv[m] = iv;
        qsum[m] = qs;
    }
};

__global__ __launch_bounds__(256) void act_quant_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps,
    int M, int K, int8_t *__restrict__ q, float *__restrict__ inv,
    int32_t *__restrict__ qsum) {
    __shared__ float red[8];
    const int m0 = blockIdx.x * 4;
    const int rows = min(4, M - m0);
    GlobalSink sink{q + (size_t)m0 * K, inv + m0, qsum + m0, K};
    block_act_quant<256>(x + (size_t)m0 * K, gamma, eps, rows, K, red, sink);
}

}  // namespace

hipError_t launch_act_quant(const float *x, const float *gamma, float eps,
                            int64_t M, int64_t K, int8_t *q, float *inv,
                            int32_t *qsum, hipStream_t s) {
    const unsigned blocks = (unsigned)((M + 3) / 4);
    hipLaunchKernelGGL(act_quant_kernel, dim3(blocks), dim3(256), 0, s, x,
                       gamma, eps, (int)M, (int)K, q, inv, qsum);
    return hipGetLastError();
}

}  // namespace bl
