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
// of fully issued loads.  Rows of 8193..32768 in launches of no more rows
// than CUs: one 1024-thread block per row (wide_act_quant_row, the same
// codes).  HBM traffic per row: 4K (x) + 4K (gamma, L2-resident after the
// first rows) + K (q) + 8 bytes.
#include <algorithm>
#include <climits>

#include "common.hpp"

namespace bl {
namespace {

struct GlobalRowSink {
    static constexpr bool kDeferSum = false;
    int8_t *q;  // row base
    float *inv;
    int32_t *qsum;
    __device__ void store_q(int k, uint32_t v) { *reinterpret_cast<uint32_t *>(q + k) = v; }
    __device__ void store_row(float iv, int qs) {
        *inv = iv;
        *qsum = qs;
    }
};

// XT: the activations' storage type (float, bf16_t, _Float16), widened to
// fp32 as they are loaded.
template <typename XT = float>
__global__ __launch_bounds__(64) void act_quant_wave_kernel(
    const XT *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    wave_act_quant_row<1, XT>(x + (size_t)m * K, gamma, eps, K, sink);
}

template <int CH, typename XT = float>
__global__ __launch_bounds__(256) void act_quant_block_kernel(
    const XT *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    __shared__ float red[kRedWords];
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    block_act_quant_row<CH, false, true, false, XT>(x + (size_t)m * K, gamma, eps, K, red, sink,
                                                    [] {});
}

template <typename XT = float>
__global__ __launch_bounds__(256) void act_quant_long_kernel(
    const XT *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    __shared__ float red[kRedWords];
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    block_act_quant_row<8, true, true, false, XT>(x + (size_t)m * K, gamma, eps, K, red, sink,
                                                  [] {});
}

// One 1024-thread block per token row (fp32 x), through wide_act_quant_row:
// the same codes as the 256-thread form with a quarter of its serial work
// per thread, for long rows in launches with no more rows than CUs (every
// row has a CU to itself, and the row's chain of dependent VALU work is the
// launch's critical path).  qsum: the sixteen per-wave code sums, order-free.
template <int SQ>
__global__ __launch_bounds__(1024) void act_quant_wide_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps, int K,
    int8_t *__restrict__ q, float *__restrict__ inv, int32_t *__restrict__ qsum) {
    __shared__ float red[20];
    __shared__ float chain[256];
    __shared__ int qpart[16];
    __shared__ float inv_sh;
    const int m = blockIdx.x;
    wide_act_quant_row<SQ, false, false>(x + (size_t)m * K, gamma, eps, K, red, chain, nullptr,
                                         q + (size_t)m * K, &inv_sh, inv + m, qpart, [] {});
    lds_barrier();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int w = 0; w < 16; ++w) t += qpart[w];
        qsum[m] = t;
    }
}

// y[m][n] = (float)acc[m][n] * (w_scale / inv[m]) rounded to the output
// type YT (bf16_t, _Float16: to nearest, ties to even, NaN kept quiet).
// Two outputs per thread.
template <typename YT>
__global__ __launch_bounds__(256) void rescale_kernel(const int32_t *__restrict__ acc,
                                                      const float *__restrict__ inv, float w_scale,
                                                      int64_t M, int64_t N, YT *__restrict__ y) {
    const int64_t total = M * N;
    const int64_t pairs = total / 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = t; i < pairs; i += stride) {
        const int64_t e = 2 * i;
        const int64_t m0 = e / N, m1 = (e + 1) / N;  // a pair may straddle two rows
        const float c0 = w_scale / inv[m0];
        const float c1 = m1 == m0 ? c0 : w_scale / inv[m1];
        const int2 a = *reinterpret_cast<const int2 *>(acc + e);
        const float v0 = (float)a.x * c0, v1 = (float)a.y * c1;
        if constexpr (std::is_same<YT, float>::value) {
            *reinterpret_cast<float2 *>(y + e) = make_float2(v0, v1);
        } else {
            *reinterpret_cast<uint32_t *>(y + e) =
                (uint32_t)to_half_bits<YT>(v0) | ((uint32_t)to_half_bits<YT>(v1) << 16);
        }
    }
    if ((total & 1) && t == 0) {  // odd element count: the last one alone
        const int64_t e = total - 1;
        const float v = (float)acc[e] * (w_scale / inv[e / N]);
        if constexpr (std::is_same<YT, float>::value)
            y[e] = v;
        else
            reinterpret_cast<uint16_t *>(y)[e] = to_half_bits<YT>(v);
    }
}

// The FFN's down-projection input: the row is relu2_mul(g, u) of the gate
// and up rows, normalised (gamma: the sub-norm) and quantised.  Rows of up
// to 1024 * CH in registers, longer ones streamed.
template <int CH, bool LONG>
__global__ __launch_bounds__(256) void act_quant_glu_kernel(
    const float *__restrict__ g, const float *__restrict__ u, const float *__restrict__ gamma,
    float eps, int K, int8_t *__restrict__ q, float *__restrict__ inv,
    int32_t *__restrict__ qsum) {
    __shared__ float red[kRedWords];
    const int m = blockIdx.x;
    GlobalRowSink sink{q + (size_t)m * K, inv + m, qsum + m};
    block_act_quant_row<CH, LONG, true, true>(g + (size_t)m * K, gamma, eps, K, red, sink, [] {},
                                              u + (size_t)m * K);
}

// a = relu2_mul(g, u) over n elements (n % 4 == 0), float4 per thread, for
// rows too long for the gated quantisation to hold in registers.
__global__ __launch_bounds__(256) void relu2_mul_kernel(const float4 *__restrict__ g,
                                                        const float4 *__restrict__ u,
                                                        float4 *__restrict__ a, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        a[i] = relu2_mul4(g[i], u[i]);
}

// Batched form: up to 8 problems, one block per token row of any of them.
// b0..b7: first block of each problem (INT_MAX past the last), leading the
// argument list so that the build's kernel-argument preload puts them in
// scalar registers at wave launch.
struct AqProblem {
    const void *x;
    const float *gamma;
    int8_t *q;
    float *inv;
    int32_t *qsum;
    float eps;
    int K;
    int row_begin;
};
constexpr int kMaxAqBatch = 8;
struct AqBatch {
    AqProblem p[kMaxAqBatch];
};

template <int CH, typename XT = float>
__global__ __launch_bounds__(256) void act_quant_batch_kernel(int b0, int b1, int b2, int b3,
                                                              int b4, int b5, int b6, int b7,
                                                              AqBatch B) {
    static_assert(kMaxAqBatch == 8, "one leading argument per problem");
    __shared__ float red[kRedWords];
    (void)b0;
    const int bx = (int)blockIdx.x;
    const int pi = (bx >= b1) + (bx >= b2) + (bx >= b3) + (bx >= b4) + (bx >= b5) + (bx >= b6) +
                   (bx >= b7);
    const AqBatch *Bk = reinterpret_cast<const AqBatch *>(
        (const char *)__builtin_amdgcn_kernarg_segment_ptr() + 8 * sizeof(int));
    const AqProblem P = Bk->p[pi];
    const int m = bx - P.row_begin;
    const int K = P.K;
    GlobalRowSink sink{P.q + (size_t)m * K, P.inv + m, P.qsum + m};
    block_act_quant_row<CH, false, true, false, XT>(static_cast<const XT *>(P.x) + (size_t)m * K,
                                                    P.gamma, P.eps, K, red, sink, [] {});
}

template <int SQ>
hipError_t launch_wide(const float *x, const float *gamma, float eps, int64_t M, int64_t K,
                       int8_t *q, float *inv, int32_t *qsum, hipStream_t s) {
    hipLaunchKernelGGL((act_quant_wide_kernel<SQ>), dim3((unsigned)M), dim3(1024), 0, s, x, gamma,
                       eps, (int)K, q, inv, qsum);
    return hipGetLastError();
}

// Whether M rows of K take the 1024-thread form: fp32 rows of 8193..32768,
// no more rows than CUs.  There the 256-thread form's per-thread chain is
// 9-32 float4 groups long (70B FFN down projection, K = 28672, M = 16:
// 32.6 -> 31.7-31.9 us per forward).  Up to K = 8192 the two forms measured the
// same (K = N = 8192 at M = 4 / 16 / 64), the launch itself dominating.
bool wide_rows(int64_t rows, int64_t K) {
    return K > 8 * 1024 && K <= 32 * 1024 && rows <= device_cus();
}

template <int CH, typename XT>
hipError_t launch_block(const XT *x, const float *gamma, float eps, int64_t M, int64_t K,
                        int8_t *q, float *inv, int32_t *qsum, hipStream_t s) {
    hipLaunchKernelGGL((act_quant_block_kernel<CH, XT>), dim3((unsigned)M), dim3(256), 0, s, x,
                       gamma, eps, (int)K, q, inv, qsum);
    return hipGetLastError();
}

template <typename XT>
hipError_t launch_act_quant_t(const XT *x, const float *gamma, float eps, int64_t M, int64_t K,
                              int8_t *q, float *inv, int32_t *qsum, hipStream_t s) {
    if (K <= 1024) {
        hipLaunchKernelGGL((act_quant_wave_kernel<XT>), dim3((unsigned)M), dim3(64), 0, s, x,
                           gamma, eps, (int)K, q, inv, qsum);
        return hipGetLastError();
    }
    if constexpr (std::is_same<XT, float>::value) {
        if (wide_rows(M, K)) {
            if (K <= 16 * 1024) return launch_wide<4>(x, gamma, eps, M, K, q, inv, qsum, s);
            return launch_wide<8>(x, gamma, eps, M, K, q, inv, qsum, s);
        }
    }
    if (K <= 4 * 1024) return launch_block<4>(x, gamma, eps, M, K, q, inv, qsum, s);
    if (K <= 8 * 1024) return launch_block<8>(x, gamma, eps, M, K, q, inv, qsum, s);
    if (K <= 16 * 1024) return launch_block<16>(x, gamma, eps, M, K, q, inv, qsum, s);
    if (K <= 32 * 1024) return launch_block<32>(x, gamma, eps, M, K, q, inv, qsum, s);
    // Rows beyond 32768: streamed in three passes.
    hipLaunchKernelGGL((act_quant_long_kernel<XT>), dim3((unsigned)M), dim3(256), 0, s, x, gamma,
                       eps, (int)K, q, inv, qsum);
    return hipGetLastError();
}

template <typename YT>
hipError_t launch_rescale_t(const int32_t *acc, const float *inv, float w_scale, int64_t M,
                            int64_t N, YT *y, hipStream_t s) {
    const int64_t pairs = (M * N + 1) / 2;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((pairs + 255) / 256, 4096));
    hipLaunchKernelGGL((rescale_kernel<YT>), dim3((unsigned)blocks), dim3(256), 0, s, acc, inv,
                       w_scale, M, N, y);
    return hipGetLastError();
}

// The fp32 arithmetic the normalisation and quantisation rest on, exposed
// elementwise so that it can be checked against correctly rounded host
// arithmetic: op 0 sqrtf(a), op 1 a / b, op 2 rms_scale(a, K = b, eps),
// op 3 quant_scale(a).  The same device functions and build flags as every
// kernel of the library.
__global__ __launch_bounds__(256) void fp32_ops_kernel(int op, const float *__restrict__ a,
                                                       const float *__restrict__ b, float eps,
                                                       int64_t n, float *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float va = a[i];
        float r;
        if (op == 0) r = sqrtf(va);
        else if (op == 1) r = va / b[i];
        else if (op == 2) r = rms_scale(va, (int)b[i], eps);
        else r = quant_scale(va);
        out[i] = r;
    }
}

}  // namespace

hipError_t launch_act_quant_batch(const ActQuantDesc *d, int count, hipStream_t s) {
    if (count < 1 || count > kMaxAqBatch) return hipErrorInvalidValue;
    AqBatch B{};
    int begin[kMaxAqBatch];
    int64_t rows = 0, kmax = 0;
    for (int i = 0; i < count; ++i) {
        if (d[i].K > kActQuantBatchMaxK || d[i].K < 1 || d[i].M < 1 || d[i].io != d[0].io)
            return hipErrorInvalidValue;
        AqProblem &P = B.p[i];
        P.x = d[i].x;
        P.gamma = d[i].gamma;
        P.q = d[i].q;
        P.inv = d[i].inv;
        P.qsum = d[i].qsum;
        P.eps = d[i].eps;
        P.K = (int)d[i].K;
        P.row_begin = (int)rows;
        begin[i] = (int)rows;
        rows += d[i].M;
        if (rows > INT32_MAX) return hipErrorInvalidConfiguration;
        kmax = std::max<int64_t>(kmax, d[i].K);
    }
    for (int i = count; i < kMaxAqBatch; ++i) begin[i] = INT32_MAX;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(256), 0, s, begin[0], begin[1],
                           begin[2], begin[3], begin[4], begin[5], begin[6], begin[7], B);
        return hipGetLastError();
    };
    const bool small = kmax <= 4096;
    switch (d[0].io) {
        case kIoF32: return small ? go(act_quant_batch_kernel<4>) : go(act_quant_batch_kernel<8>);
        case kIoBf16:
            return small ? go(act_quant_batch_kernel<4, bf16_t>) : go(act_quant_batch_kernel<8, bf16_t>);
        case kIoF16:
            return small ? go(act_quant_batch_kernel<4, _Float16>)
                         : go(act_quant_batch_kernel<8, _Float16>);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_act_quant_glu(const float *g, const float *u, const float *gamma, float eps,
                                int64_t M, int64_t K, int8_t *q, float *inv, int32_t *qsum,
                                hipStream_t s) {
    const dim3 grid((unsigned)M), block(256);
    if (K <= 4 * 1024)
        hipLaunchKernelGGL((act_quant_glu_kernel<4, false>), grid, block, 0, s, g, u, gamma, eps,
                           (int)K, q, inv, qsum);
    else if (K <= 8 * 1024)
        hipLaunchKernelGGL((act_quant_glu_kernel<8, false>), grid, block, 0, s, g, u, gamma, eps,
                           (int)K, q, inv, qsum);
    else
        hipLaunchKernelGGL((act_quant_glu_kernel<8, true>), grid, block, 0, s, g, u, gamma, eps,
                           (int)K, q, inv, qsum);
    return hipGetLastError();
}

hipError_t launch_relu2_mul(const float *g, const float *u, float *a, int64_t n, hipStream_t s) {
    const int64_t n4 = n / 4;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n4 + 255) / 256, 4096));
    hipLaunchKernelGGL(relu2_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(g), reinterpret_cast<const float4 *>(u),
                       reinterpret_cast<float4 *>(a), n4);
    return hipGetLastError();
}

hipError_t launch_act_quant(const float *x, const float *gamma, float eps,
                            int64_t M, int64_t K, int8_t *q, float *inv,
                            int32_t *qsum, hipStream_t s) {
    return launch_act_quant_t(x, gamma, eps, M, K, q, inv, qsum, s);
}

hipError_t launch_act_quant_io(const void *x, int xtype, const float *gamma, float eps, int64_t M,
                               int64_t K, int8_t *q, float *inv, int32_t *qsum, hipStream_t s) {
    switch (xtype) {
        case kIoF32:
            return launch_act_quant_t(static_cast<const float *>(x), gamma, eps, M, K, q, inv,
                                      qsum, s);
        case kIoBf16:
            return launch_act_quant_t(static_cast<const bf16_t *>(x), gamma, eps, M, K, q, inv,
                                      qsum, s);
        case kIoF16:
            return launch_act_quant_t(static_cast<const _Float16 *>(x), gamma, eps, M, K, q, inv,
                                      qsum, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rescale_io(const int32_t *acc, const float *inv, float w_scale, int64_t M,
                             int64_t N, void *y, int ytype, hipStream_t s) {
    switch (ytype) {
        case kIoF32:
            return launch_rescale_t(acc, inv, w_scale, M, N, static_cast<float *>(y), s);
        case kIoBf16:
            return launch_rescale_t(acc, inv, w_scale, M, N, static_cast<bf16_t *>(y), s);
        case kIoF16:
            return launch_rescale_t(acc, inv, w_scale, M, N, static_cast<_Float16 *>(y), s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fp32_ops(int op, const float *a, const float *b, float eps, int64_t n,
                           float *out, hipStream_t s) {
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 8192));
    hipLaunchKernelGGL(fp32_ops_kernel, dim3((unsigned)blocks), dim3(256), 0, s, op, a, b, eps, n,
                       out);
    return hipGetLastError();
}

}  // namespace bl
