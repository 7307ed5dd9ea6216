// gemv.hip -- decode route of the ternary x int8 contraction (gfx950).
//
// acc[m][n] = sum_k code(n, k) * q[m][k] - qsum[m], then optionally
// y[m][n] = (float)acc * (w_scale / inv[m]).
// [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU FFN":
// the vec_dot over I2_S codes and int8 activations, codes offset by the
// activation sum; every output must be written.]
//
// Design.  Decode is bound by streaming the packed weights (N*K/4 bytes)
// from HBM once, so the kernel is built around full-line loads and
// memory-level parallelism:
//  - Lane l loads 16 packed bytes of row l % 8 at chunk l / 8 of a 128-byte
//    step: one global load per wave covers 8 rows x 128 bytes, i.e. whole
//    128-byte cache lines (a 16-row x 64-byte pattern streams ~30% slower).
//    Each wave issues U steps per batch and prefetches the next batch before
//    contracting the current one (double-buffered registers).
//  - The 16 bytes hold, per 2-bit field g, the codes of 16 consecutive k.
//    They go, shifted and masked, straight into v_mfma_i32_16x16x64_i8 as the
//    B operand: the 16 MFMA columns are 8 weight rows x 2 chunk parities.
//    The A operand repeats each token in both halves of the 16 rows with the
//    matching chunk, so D block (tokens 0-7, columns 0-7) holds the even
//    chunks' dot products and block (tokens 8-15, columns 8-15) the odd
//    chunks'; one lane + 40 add joins them.  The other blocks are unused --
//    the MFMA pipe has ample headroom at decode.  Tokens 8-15 take a second
//    MFMA (TH = 2).  One independent accumulator per field.
//  - The K range of a tile group (R tiles of 8 rows) is split over the 4
//    waves; the int32 partial tiles are summed through LDS (exact, order-
//    free) and the epilogue subtracts qsum and rescales.
//  - Workgroups walk tile groups with a grid stride, so per-workgroup set-up
//    (the fused quantisation below) is paid once per workgroup, and the next
//    tile group's weights are already in flight during the reduction.
// Activation operand (MODE):
//  0 fused: every workgroup recomputes RMSNorm + int8 quantisation of its
//    (<= 4) token rows into LDS while its first weight loads are in flight,
//    so a decode BitLinear is one launch; workgroup 0 also writes q / inv /
//    qsum to the workspace.  Bit-identical to the separate kernel (same
//    arithmetic, same order).
//  1 staged: the token group's q rows are copied into LDS once.
//  2 global: q fragments are loaded from global memory (L2) per batch.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kW = 4;           // waves per workgroup
constexpr int kTileRows = 8;    // weight rows per tile
constexpr int kStep = 128;      // packed bytes of a row per step (512 k)

struct LdsRowSink {
    int8_t *q;
    float *inv;
    int *qsum;
    __device__ void store_q(int k, uint32_t v) { *reinterpret_cast<uint32_t *>(q + k) = v; }
    __device__ void store_row(float iv, int qs) {
        *inv = iv;
        *qsum = qs;
    }
};

// FM (MODE 0): compile-time bound on the token rows (M <= FM); LONG
// (MODE 0): rows longer than 8192 take the streamed normalisation.  TH:
// token halves (1 for M <= 8, 2 for M <= 16).
template <int R, int U, int MODE, bool OUT_Y, int FM, bool LONG, int TH>
__global__ __launch_bounds__(256) void gemv_kernel(
    const float *__restrict__ x, const float *__restrict__ gamma, float eps,
    const int8_t *__restrict__ q, const float *__restrict__ inv,
    const int32_t *__restrict__ qsum, const uint8_t *__restrict__ packed,
    float w_scale, int M, int K, int N, float *__restrict__ y,
    int32_t *__restrict__ acc_out, int8_t *__restrict__ q_out,
    float *__restrict__ inv_out, int32_t *__restrict__ qsum_out) {
    extern __shared__ __align__(16) int8_t q_lds[];
    __shared__ float red[4];
    __shared__ float inv_sh[4];
    __shared__ int qsum_sh[4];
    __shared__ v4i part[kW][TH][R][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int r8 = lane & 7;    // weight row within the tile (load role)
    const int ch = lane >> 3;   // 16-byte chunk within the 128-byte step
    const int m0 = MODE == 0 ? 0 : blockIdx.y * 16;
    const int mg = min(16, M - m0);  // tokens of this workgroup's group

    const uint32_t rowbytes = (uint32_t)K / 4;
    const int nsteps = (int)((rowbytes + kStep - 1) / kStep);
    const int nb = (nsteps + kW * U - 1) / (kW * U);
    const int ntg = (N + kTileRows * R - 1) / (kTileRows * R);
    // MODE 2: q rows of this token group, range-checked.
    const auto rq = make_rsrc(q + (size_t)m0 * K, (uint32_t)(mg * K));

    v4i bcur[U][R], bnxt[U][R];
    v4i acc[4][TH][R];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h = 0; h < TH; ++h)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[g][h][r] = v4i{0, 0, 0, 0};

    int tg = blockIdx.x;
    int b = 0;

    // Weights of batch b_ of tile group tg_ (wave w takes steps
    // b_*W*U + w*U + [0, U)); rows past N and bytes past the row read zero.
    auto load_batch = [&](v4i(&buf)[U][R], int tg_, int b_) {
        const int n0 = tg_ * kTileRows * R;
        const int rows = min(kTileRows * R, N - n0);
        const auto rw = make_rsrc(packed + (size_t)n0 * rowbytes, (uint32_t)rows * rowbytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = b_ * kW * U + wid * U + u;
            const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
            const bool kv = (s < nsteps) && (cb < rowbytes);
#pragma unroll
            for (int r = 0; r < R; ++r)
                buf[u][r] = buf_load16(rw, kv ? (uint32_t)(kTileRows * r + r8) * rowbytes + cb : kOOB);
        }
    };

    if constexpr (MODE == 0) {
        // x and gamma loads go first, the first weight batch right behind
        // them, so the normalisation never waits for the weights.
        {
            LdsRowSink sink{q_lds, inv_sh, qsum_sh};
            block_act_quant_row<8, LONG>(x, gamma, eps, K, red, sink,
                                         [&] { load_batch(bcur, tg, b); });
        }
#pragma unroll
        for (int m = 1; m < FM; ++m) {
            if (m < M) {
                LdsRowSink sink{q_lds + m * K, inv_sh + m, qsum_sh + m};
                block_act_quant_row<8, LONG>(x + (size_t)m * K, gamma, eps, K, red, sink, [] {});
            }
        }
        __syncthreads();
        if (blockIdx.x == 0) {
            for (int i = tid; i < M * K / 16; i += 256)
                reinterpret_cast<uint4 *>(q_out)[i] = reinterpret_cast<const uint4 *>(q_lds)[i];
            if (tid < M) {
                inv_out[tid] = inv_sh[tid];
                qsum_out[tid] = qsum_sh[tid];
            }
        }
    } else if constexpr (MODE == 1) {
        const uint4 *src = reinterpret_cast<const uint4 *>(q + (size_t)m0 * K);
        for (int i = tid; i < mg * K / 16; i += 256)
            reinterpret_cast<uint4 *>(q_lds)[i] = src[i];
        load_batch(bcur, tg, b);
        __syncthreads();
    } else {
        load_batch(bcur, tg, b);
    }

    for (;;) {
        int tg2 = tg, b2 = b + 1;
        if (b2 == nb) {
            tg2 += gridDim.x;
            b2 = 0;
        }
        const bool more = tg2 < ntg;
        if (more) load_batch(bnxt, tg2, b2);

        // Contract the current batch.
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = b * kW * U + wid * U + u;
            const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
            const bool kv = (s < nsteps) && (cb < rowbytes);
            // k of this lane's chunk: block cb / 32, half (cb / 16) % 2.
            const int kb = (int)(cb / 32) * kBlockWeights + 16 * (int)((cb / 16) & 1);
            v4i a[TH][4];
#pragma unroll
            for (int h = 0; h < TH; ++h) {
                const int t = 8 * h + r8;  // token (group-relative)
                const bool av = kv && t < mg;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if constexpr (MODE == 2) {
                        a[h][g] = buf_load16(rq, av ? (uint32_t)(t * K + kb + 32 * g) : kOOB);
                    } else {
                        a[h][g] = av ? *reinterpret_cast<const v4i *>(q_lds + t * K + kb + 32 * g)
                                     : v4i{0, 0, 0, 0};
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const v4i bf = unpack_field(bcur[u][r], g);
#pragma unroll
                    for (int h = 0; h < TH; ++h) acc[g][h][r] = mfma16(a[h][g], bf, acc[g][h][r]);
                }
        }

        if (b == nb - 1) {
            // Tile group done: sum the fields, then the waves' partials.
#pragma unroll
            for (int h = 0; h < TH; ++h)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    part[wid][h][r][lane] =
                        (acc[0][h][r] + acc[1][h][r]) + (acc[2][h][r] + acc[3][h][r]);
#pragma unroll
                    for (int g = 0; g < 4; ++g) acc[g][h][r] = v4i{0, 0, 0, 0};
                }
            __syncthreads();
            // D(i, j) lives in lane j + 16*(i/4), register i%4.  Useful
            // lanes: [0, 8) and [16, 24) (even chunks, rows j, tokens
            // 4*(lane/16) + c) and lane + 40 (odd chunks, same rows/tokens).
            for (int hr = wid; hr < TH * R; hr += kW) {
                const int h = hr / R, r = hr % R;
                const int l = lane;
                const bool useful = (l & 8) == 0 && l < 24;
                if (useful) {
                    v4i t = part[0][h][r][l] + part[0][h][r][l + 40];
#pragma unroll
                    for (int w = 1; w < kW; ++w) t += part[w][h][r][l] + part[w][h][r][l + 40];
                    const int n = tg * kTileRows * R + kTileRows * r + (l & 7);
                    if (n < N) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int mloc = 8 * h + 4 * (l >> 4) + c;
                            if (mloc < mg) {
                                const int m = m0 + mloc;
                                const int qs = MODE == 0 ? qsum_sh[m] : qsum[m];
                                const int v = t[c] - qs;
                                if (OUT_Y) {
                                    const float iv = MODE == 0 ? inv_sh[m] : inv[m];
                                    y[(size_t)m * N + n] = (float)v * (w_scale / iv);
                                } else {
                                    acc_out[(size_t)m * N + n] = v;
                                }
                            }
                        }
                    }
                }
            }
            __syncthreads();
        }
        if (!more) break;
        tg = tg2;
        b = b2;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r) bcur[u][r] = bnxt[u][r];
    }
}

struct Shape {
    int R, U;
};
// Launch-shape table; every entry computes bit-identical results.
constexpr Shape kShapes[] = {{2, 4}, {1, 4}, {1, 2}, {2, 2}, {4, 2}, {1, 8}};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// Workgroups of `kernel` that fit on one CU at once with `lds` dynamic LDS
// bytes (at least 1).
template <class Kern>
int resident_per_cu(Kern kernel, size_t lds) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, lds) != hipSuccess || n < 1)
        return 1;
    return n;
}

template <int R, int U, int MODE, bool OUT_Y, int FM, bool LONG, int TH>
hipError_t launch_one(const float *x, const float *gamma, float eps, const int8_t *q,
                      const float *inv, const int32_t *qsum, const uint8_t *packed,
                      float w_scale, int64_t M, int64_t K, int64_t N, float *y, int32_t *acc,
                      hipStream_t s) {
    const int64_t ntg = (N + kTileRows * R - 1) / (kTileRows * R);
    const unsigned gy = MODE == 0 ? 1u : (unsigned)((M + 15) / 16);
    const int64_t mg = M < 16 ? M : 16;
    const size_t lds = MODE == 0 ? (size_t)(M * K) : MODE == 1 ? (size_t)(mg * K) : 0;
    // One wave of co-resident workgroups walks all tile groups: per-
    // workgroup set-up is paid once and no workgroup starts late.
    auto kern = gemv_kernel<R, U, MODE, OUT_Y, FM, LONG, TH>;
    const int64_t cap = (int64_t)cu_count() * resident_per_cu(kern, lds) / gy;
    const unsigned gx = (unsigned)(ntg < cap ? ntg : (cap > 0 ? cap : 1));
    // With MODE 0, q / inv / qsum are outputs (the caller's workspace).
    hipLaunchKernelGGL((gemv_kernel<R, U, MODE, OUT_Y, FM, LONG, TH>), dim3(gx, gy), dim3(256),
                       lds, s, x, gamma, eps, q, inv, qsum, packed, w_scale, (int)M, (int)K,
                       (int)N, y, acc, const_cast<int8_t *>(q), const_cast<float *>(inv),
                       const_cast<int32_t *>(qsum));
    return hipGetLastError();
}

template <int R, int U>
hipError_t launch_shape(const float *x, const float *gamma, float eps, const int8_t *q,
                        const float *inv, const int32_t *qsum, const uint8_t *packed,
                        float w_scale, int64_t M, int64_t K, int64_t N, float *y, int32_t *acc,
                        int mode, hipStream_t s) {
    if (mode == 0) {  // forward only: y is always written; M <= 4 so TH = 1
        const bool lng = K > 8 * 1024;
        if (M == 1)
            return lng ? launch_one<R, U, 0, true, 1, true, 1>(x, gamma, eps, q, inv, qsum, packed,
                                                               w_scale, M, K, N, y, acc, s)
                       : launch_one<R, U, 0, true, 1, false, 1>(x, gamma, eps, q, inv, qsum,
                                                                packed, w_scale, M, K, N, y, acc,
                                                                s);
        return lng ? launch_one<R, U, 0, true, kFuseMaxM, true, 1>(x, gamma, eps, q, inv, qsum,
                                                                   packed, w_scale, M, K, N, y,
                                                                   acc, s)
                   : launch_one<R, U, 0, true, kFuseMaxM, false, 1>(x, gamma, eps, q, inv, qsum,
                                                                    packed, w_scale, M, K, N, y,
                                                                    acc, s);
    }
#define BL_ONE(MODE, TH)                                                                        \
    return y ? launch_one<R, U, MODE, true, 0, false, TH>(x, gamma, eps, q, inv, qsum, packed,    \
                                                          w_scale, M, K, N, y, acc, s)            \
             : launch_one<R, U, MODE, false, 0, false, TH>(x, gamma, eps, q, inv, qsum, packed,   \
                                                           w_scale, M, K, N, y, acc, s);
    const bool two = M > 8;
    if (mode == 1) {
        if (two) { BL_ONE(1, 2) }
        BL_ONE(1, 1)
    }
    if (two) { BL_ONE(2, 2) }
    BL_ONE(2, 1)
#undef BL_ONE
}

}  // namespace

int gemv_num_variants() { return kNumShapes; }

hipError_t launch_gemv(const float *x, const float *gamma, float eps,
                       const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, int64_t N, float *y, int32_t *acc,
                       bool fused, int variant, hipStream_t s) {
    const int64_t mg = M < 16 ? M : 16;
    const int mode = fused ? 0 : (mg * K <= kGemvStageMaxLds ? 1 : 2);
    int v = variant;
    if (v <= 0) {
        // One batch of U 128-byte steps per wave covers rows up to 4*U*128 bytes.
        const int64_t nsteps = (K / 4 + kStep - 1) / kStep;
        v = nsteps > 8 ? 1 : 3;
    }
#define BL_GEMV_CASE(idx)                                                                   \
    case idx:                                                                               \
        return launch_shape<kShapes[idx - 1].R, kShapes[idx - 1].U>(                        \
            x, gamma, eps, q, inv, qsum, packed, w_scale, M, K, N, y, acc, mode, s);
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
