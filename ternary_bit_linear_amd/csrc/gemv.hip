// gemv.hip -- decode route of the ternary x int8 contraction (gfx950).
//
// acc[m][n] = sum_k code(n, k) * q[m][k] - qsum[m], then optionally
// y[m][n] = (float)acc * (w_scale / inv[m]).
// [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU FFN":
// the vec_dot over I2_S codes and int8 activations, codes offset by the
// activation sum; every output must be written.]
//
// Design.  Decode is bound by streaming the packed weights (N*K/4 bytes)
// from HBM once.  Each lane loads 16 packed bytes (64 weights of one row)
// per step with one global_load_dwordx4; the 16 lanes that share a k-group
// cover 16 rows, the 4 k-groups cover 64 contiguous bytes of each row.  The
// codes are expanded in registers (shift + mask per field) and fed to
// v_mfma_i32_16x16x64_i8 with the tokens (up to 16) as the other operand,
// so the per-weight VALU work is one shift+mask per 4 weights whatever M is.
// The K loop of a 16-row tile is split over the W waves of a workgroup
// (interleaved 64-byte steps), and the W partial int32 tiles are summed in
// LDS (integer sums: exact, order-free).  With `FUSED`, every workgroup
// first recomputes the RMSNorm + int8 quantisation of its (<= 4) token rows
// into LDS -- x and gamma come from L2 -- so decode is a single launch.
#include "common.hpp"

namespace bl {
namespace {

struct LdsSink {
    int8_t *q;
    float *inv;
    int *qsum;
    int K;
    __device__ void store_q(int m, int k, uint32_t v) {
        *reinterpret_cast<uint32_t *>(q + m * K + k) = v;
    }
    __device__ void store_row(int m, float iv, int qs) {
        inv[m] = iv;
        qsum[m] = qs;
    }
};

__device__ __forceinline__ uint4 load16(const uint8_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// W waves per workgroup, R 16-row tiles per workgroup, U steps per wave in
// flight.
template <int W, int R, int U, bool FUSED, bool OUT_Y>
__global__ __launch_bounds__(W * 64) void gemv_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps,
    const int8_t *__restrict__ q, const float *__restrict__ inv,
    const int32_t *__restrict__ qsum, const uint8_t *__restrict__ packed,
    float w_scale, int M, int K, int N, float *__restrict__ y,
    int32_t *__restrict__ acc_out, int8_t *__restrict__ q_out,
    float *__restrict__ inv_out, int32_t *__restrict__ qsum_out) {
    static_assert(R <= W, "one reduction tile per wave");
    extern __shared__ __align__(16) int8_t q_lds[];
    __shared__ float red_sh[16];
    __shared__ float inv_sh[4];
    __shared__ int qsum_sh[4];
    __shared__ v4i part[W][R][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int j = lane & 15;   // A row (token) / B column (weight row) slot
    const int kg = lane >> 4;  // k-group of the lane
    const int m0 = FUSED ? 0 : blockIdx.y * 16;
    const int n0 = blockIdx.x * 16 * R;

    if (FUSED) {
        LdsSink sink{q_lds, inv_sh, qsum_sh, K};
        block_act_quant<W * 64>(x, gamma, eps, M, K, red_sh, sink);
        // Workgroup 0 also leaves q / inv / qsum in the caller's workspace.
        if (blockIdx.x == 0) {
            for (int i = tid; i < M * K / 16; i += W * 64)
                reinterpret_cast<uint4 *>(q_out)[i] = reinterpret_cast<const uint4 *>(q_lds)[i];
            if (tid < M) {
                inv_out[tid] = inv_sh[tid];
                qsum_out[tid] = qsum_sh[tid];
            }
        }
    }

    const int nsteps = (K + kStepK - 1) / kStepK;
    const int nblocks = K / kBlockWeights;
    const size_t rowbytes = (size_t)K / 4;

    const uint8_t *brow[R];
    bool bval[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int n = n0 + 16 * r + j;
        bval[r] = n < N;
        brow[r] = packed + (size_t)(bval[r] ? n : 0) * rowbytes + 16 * kg;
    }
    const int mi = m0 + j;
    const bool aval = mi < M;
    const int8_t *arow = FUSED ? (q_lds + (aval ? j : 0) * K)
                               : (q + (size_t)(aval ? mi : 0) * K);

    v4i acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = v4i{0, 0, 0, 0};

    for (int s0 = wid; s0 < nsteps; s0 += W * U) {
        uint4 b[U][R];
        bool kv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * W;
            kv[u] = (s < nsteps) && (2 * s + (kg >> 1) < nblocks);
#pragma unroll
            for (int r = 0; r < R; ++r)
                b[u][r] = (kv[u] && bval[r]) ? load16(brow[r] + (size_t)s * kStepBytes)
                                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * W;
            const int kb = (2 * s + (kg >> 1)) * kBlockWeights + 16 * (kg & 1);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                v4i a = v4i{0, 0, 0, 0};
                if (kv[u] && aval) a = *reinterpret_cast<const v4i *>(arow + kb + 32 * g);
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = mfma16(a, unpack_field(b[u][r], g), acc[r]);
            }
        }
    }

    // Sum the W partial tiles.
#pragma unroll
    for (int r = 0; r < R; ++r) part[wid][r][lane] = acc[r];
    __syncthreads();
    for (int r = wid; r < R; r += W) {
        v4i t = part[0][r][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) t += part[w][r][lane];
        const int n = n0 + 16 * r + j;
        if (n < N) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int m = m0 + 4 * kg + c;
                if (m < M) {
                    const int qs = FUSED ? qsum_sh[m] : qsum[m];
                    const int v = t[c] - qs;
                    if (OUT_Y) {
                        const float iv = FUSED ? inv_sh[m] : inv[m];
                        y[(size_t)m * N + n] = (float)v * (w_scale / iv);
                    } else {
                        acc_out[(size_t)m * N + n] = v;
                    }
                }
            }
        }
    }
}

struct Shape {
    int W, R, U;
};
// Launch-shape table; every entry computes bit-identical results.
constexpr Shape kShapes[] = {{4, 1, 2}, {4, 2, 2}, {8, 1, 2}, {4, 4, 1}, {8, 2, 1}, {4, 1, 4}};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

template <int W, int R, int U, bool FUSED, bool OUT_Y>
hipError_t launch_one(const float *x, const float *gamma, float eps,
                      const int8_t *q, const float *inv, const int32_t *qsum,
                      const uint8_t *packed, float w_scale, int64_t M, int64_t K,
                      int64_t N, float *y, int32_t *acc, hipStream_t s) {
    const unsigned gx = (unsigned)((N + 16 * R - 1) / (16 * R));
    const unsigned gy = FUSED ? 1u : (unsigned)((M + 15) / 16);
    const size_t lds = FUSED ? (size_t)M * (size_t)K : 0;
    // In the fused form q / inv / qsum are outputs (the caller's workspace).
    hipLaunchKernelGGL((gemv_kernel<W, R, U, FUSED, OUT_Y>), dim3(gx, gy), dim3(W * 64), lds,
                       s, x, gamma, eps, q, inv, qsum, packed, w_scale, (int)M,
                       (int)K, (int)N, y, acc, const_cast<int8_t *>(q),
                       const_cast<float *>(inv), const_cast<int32_t *>(qsum));
    return hipGetLastError();
}

template <int W, int R, int U>
hipError_t launch_shape(const float *x, const float *gamma, float eps,
                        const int8_t *q, const float *inv, const int32_t *qsum,
                        const uint8_t *packed, float w_scale, int64_t M, int64_t K,
                        int64_t N, float *y, int32_t *acc, bool fused, hipStream_t s) {
    if (fused)
        return y ? launch_one<W, R, U, true, true>(x, gamma, eps, q, inv, qsum, packed, w_scale, M, K, N, y, acc, s)
                 : launch_one<W, R, U, true, false>(x, gamma, eps, q, inv, qsum, packed, w_scale, M, K, N, y, acc, s);
    return y ? launch_one<W, R, U, false, true>(x, gamma, eps, q, inv, qsum, packed, w_scale, M, K, N, y, acc, s)
             : launch_one<W, R, U, false, false>(x, gamma, eps, q, inv, qsum, packed, w_scale, M, K, N, y, acc, s);
}

}  // namespace

int gemv_num_variants() { return kNumShapes; }

hipError_t launch_gemv(const float *x, const float *gamma, float eps,
                       const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, int64_t N, float *y, int32_t *acc,
                       bool fused, int variant, hipStream_t s) {
    int v = variant;
    if (v <= 0) v = 1;
#define BL_GEMV_CASE(idx)                                                          \
    case idx:                                                                      \
        return launch_shape<kShapes[idx - 1].W, kShapes[idx - 1].R, kShapes[idx - 1].U>( \
            x, gamma, eps, q, inv, qsum, packed, w_scale, M, K, N, y, acc, fused, s);
    switch (v) {
        BL_GEMV_CASE(1)
        BL_GEMV_CASE(2)
        BL_GEMV_CASE(3)
        BL_GEMV_CASE(4)
        BL_GEMV_CASE(5)
        BL_GEMV_CASE(6)
        default:
            return hipErrorInvalidValue;
    }
#undef BL_GEMV_CASE
}

}  // namespace bl
