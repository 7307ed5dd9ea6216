// act_quant.hip -- RMSNorm + per-token absmax int8 quantisation (gfx950).
//
// [huggingface/transformers PR #38087 "Add optional RMSNorm support to BitNet
// quantization (config + layers)", "What does this PR do?": the BitNet
// RMSNorm (eps default 1e-6) runs on the activations before quantisation.]
// [eejd/cpp-bitnet PR #7, NEON-kernel commit: the activations enter the
// ternary dot product as int8 together with their sum.]
//
// One wave per token row (wave_act_quant_row): every load of x and gamma is
// issued at once through range-checked buffer loads, reductions are wave
// shuffles only (no LDS, no barrier).  Rows up to 3072 elements are read
// once; longer rows take three passes (the second and third from L2).  HBM
// traffic per row: 4K (x) + 4K (gamma, L2-resident after the first rows) +
// K (q) + 8 bytes.
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

__global__ __launch_bounds__(64) void act_quant_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    wave_act_quant_row<3>(x + (size_t)m * K, gamma, eps, K, sink);
}

}  // namespace

hipError_t launch_act_quant(const float *x, const float *gamma, float eps,
                            int64_t M, int64_t K, int8_t *q, float *inv,
                            int32_t *qsum, hipStream_t s) {
    hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)M), dim3(64), 0, s, x, gamma, eps,
                       (int)K, q, inv, qsum);
    return hipGetLastError();
}

}  // namespace bl
