// gemm.hip -- prefill route of the ternary x int8 contraction (gfx950).
//
// acc[m][n] = sum_k code(n, k) * q[m][k] - qsum[m], then optionally
// y[m][n] = (float)acc * (w_scale / inv[m]).
// [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU FFN":
// the prompt-processing GEMM over I2_S codes and int8 activations, which
// must write every output; codes offset by the activation sum.]
//
// Design.  A workgroup owns a BM x BN output tile (tokens x weight rows) and
// walks K in stages of KSUB x 256 (two I2_S blocks per 256).  Per stage the
// int8 activation tile (BM x 256 KSUB) is staged in LDS with coalesced 16-byte loads (rows padded
// by 16 bytes so the 16 lanes of an MFMA row-group hit distinct banks);
// the packed weights go straight from global memory to registers -- one
// 16-byte load per lane per 16 weight rows, i.e. 64 weights -- and are
// expanded there by shift+mask into the int8 B operand of
// v_mfma_i32_16x16x64_i8 (codes 0/1/2; the activation sum is subtracted in
// the epilogue).  Each wave computes a (BM/WM) x (BN/WN) sub-tile with
// int32 accumulators in registers.  All loads are range-checked buffer
// loads (ragged M, N and K tails read zeros) issued a full step ahead of
// their use: LDS is double-buffered, one barrier per stage.
#include "common.hpp"

namespace bl {
namespace {

// BM x BN output tile per workgroup, WM x WN waves; each pipeline stage
// covers KSUB 256-k steps (KSUB * 256 bytes of every activation row).
template <int BM, int BN, int WM, int WN, int KSUB, bool OUT_Y>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ inv,
    const int32_t *__restrict__ qsum, const uint8_t *__restrict__ packed,
    float w_scale, int M, int K, int N, float *__restrict__ y,
    int32_t *__restrict__ acc_out) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MI = TM / 16, NI = TN / 16;
    constexpr int KST = kStepK * KSUB;            // k (= activation bytes) per stage
    constexpr int LROW = KST + 16;                // padded LDS row
    constexpr int CH = BM * (KST / 16) / NT;      // 16-byte A chunks per thread per stage
    static_assert(BM * (KST / 16) % NT == 0, "A tile chunks per thread");
    __shared__ __align__(16) int8_t a_lds[2][BM * LROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int j = lane & 15, kg = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;

    const int nstages = (K + KST - 1) / KST;
    const int nblocks = K / kBlockWeights;
    const uint32_t rowbytes = (uint32_t)K / 4;
    // Range-checked views of this tile's activation rows and weight rows:
    // rows past M or N read as zero.
    const auto rq = make_rsrc(q + (size_t)m0 * K, (uint32_t)min(BM, M - m0) * (uint32_t)K);
    const auto rw = make_rsrc(packed + (size_t)n0 * rowbytes,
                              (uint32_t)min(BN, N - n0) * rowbytes);

    auto load_a = [&](v4i(&areg)[CH], int st) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            const int row = idx / (KST / 16);
            const int k = st * KST + (idx % (KST / 16)) * 16;
            areg[c] = buf_load16(rq, k < K ? (uint32_t)row * (uint32_t)K + (uint32_t)k : kOOB);
        }
    };
    auto store_a = [&](int8_t *lds, const v4i(&areg)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            const int row = idx / (KST / 16);
            const int col = (idx % (KST / 16)) * 16;
            *reinterpret_cast<v4i *>(lds + row * LROW + col) = areg[c];
        }
    };
    // B of stage st: for each 256-k step t of the stage and each 16-row
    // group ni, 16 packed bytes per lane (row j, block-pair bytes 16*kg).
    auto load_b = [&](v4i(&breg)[KSUB][NI], int st) {
#pragma unroll
        for (int t = 0; t < KSUB; ++t) {
            const int s = st * KSUB + t;
            const bool kv = 2 * s + (kg >> 1) < nblocks;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const uint32_t row = (uint32_t)(wn * TN + 16 * ni + j);
                breg[t][ni] = buf_load16(rw, kv ? row * rowbytes + (uint32_t)s * kStepBytes + 16u * kg
                                                : kOOB);
            }
        }
    };

    v4i acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4i{0, 0, 0, 0};

    const int koff = (kg >> 1) * kBlockWeights + 16 * (kg & 1);
    // One 256-k step t of a stage: the step's A fragments are read from LDS
    // up front, then per field the B codes are expanded and the MI x NI
    // MFMAs issued.
    auto compute = [&](const int8_t *lds, const v4i(&breg)[KSUB][NI]) {
#pragma unroll
        for (int t = 0; t < KSUB; ++t) {
            v4i a[4][MI];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    a[g][mi] = *reinterpret_cast<const v4i *>(
                        lds + (wm * TM + 16 * mi + j) * LROW + kStepK * t + koff + 32 * g);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                v4i bf[NI];
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) bf[ni] = unpack_field(breg[t][ni], g);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni)
                        acc[mi][ni] = mfma16(a[g][mi], bf[ni], acc[mi][ni]);
            }
        }
    };

    // Software pipeline: while stage st is contracted from one LDS buffer,
    // the loads of stage st + 1 are in flight; they are written to the other
    // buffer afterwards, and one barrier per stage separates the two.
    v4i areg[CH], bcur[KSUB][NI], bnxt[KSUB][NI];
    load_a(areg, 0);
    load_b(bcur, 0);
    store_a(a_lds[0], areg);
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
        int8_t *cur = a_lds[st & 1];
        int8_t *nxt = a_lds[(st & 1) ^ 1];
        const bool more = st + 1 < nstages;
        if (more) {
            load_a(areg, st + 1);
            load_b(bnxt, st + 1);
        }
        compute(cur, bcur);
        if (more) store_a(nxt, areg);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < KSUB; ++t)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bcur[t][ni] = bnxt[t][ni];
    }

    // Epilogue: D(i, j) of a 16x16 tile is lane j + 16*(i/4), register i%4.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = m0 + wm * TM + 16 * mi + 4 * kg + c;
            if (m >= M) continue;
            const int qs = qsum[m];
            const float sc = OUT_Y ? (w_scale / inv[m]) : 0.0f;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int n = n0 + wn * TN + 16 * ni + j;
                if (n >= N) continue;
                const int v = acc[mi][ni][c] - qs;
                if (OUT_Y)
                    y[(size_t)m * N + n] = (float)v * sc;
                else
                    acc_out[(size_t)m * N + n] = v;
            }
        }
    }
}

struct Tile {
    int BM, BN, WM, WN, KSUB;
};
// Launch-shape table; every entry computes bit-identical results.
constexpr Tile kTiles[] = {{64, 128, 1, 4, 1}, {64, 128, 1, 4, 2}, {64, 128, 1, 4, 4},
                           {64, 64, 2, 2, 1},  {64, 64, 2, 2, 2},  {64, 64, 2, 2, 4},
                           {128, 128, 2, 2, 1}, {128, 128, 2, 2, 2}, {32, 64, 1, 4, 4}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <int BM, int BN, int WM, int WN, int KSUB>
hipError_t launch_tile(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M, int64_t K,
                       int64_t N, float *y, int32_t *acc, hipStream_t s) {
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    const dim3 block(WM * WN * 64);
    if (y)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KSUB, true>), grid, block, 0, s, q, inv,
                           qsum, packed, w_scale, (int)M, (int)K, (int)N, y, acc);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KSUB, false>), grid, block, 0, s, q, inv,
                           qsum, packed, w_scale, (int)M, (int)K, (int)N, y, acc);
    return hipGetLastError();
}

}  // namespace

int gemm_num_variants() { return kNumTiles; }

hipError_t launch_gemm(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, int64_t N, float *y, int32_t *acc,
                       int variant, hipStream_t s) {
    int v = variant;
    if (v <= 0) {
        // Measured on MI355X: large grids prefer the 64x128 tile (two 256-k
        // steps per stage once the grid is under ~4 waves of workgroups);
        // smaller ones trade tile size for workgroups and a deeper stage.
        auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
        v = tiles(64, 128) >= 1024 ? 1 : tiles(64, 128) >= 384 ? 2 : tiles(64, 64) >= 256 ? 5 : 9;
    }
#define BL_GEMM_CASE(idx)                                                               \
    case idx:                                                                           \
        return launch_tile<kTiles[idx - 1].BM, kTiles[idx - 1].BN, kTiles[idx - 1].WM,  \
                           kTiles[idx - 1].WN, kTiles[idx - 1].KSUB>(q, inv, qsum, packed, \
                                                                     w_scale, M, K, N, y, acc, s);
    switch (v) {
        BL_GEMM_CASE(1)
        BL_GEMM_CASE(2)
        BL_GEMM_CASE(3)
        BL_GEMM_CASE(4)
        BL_GEMM_CASE(5)
        BL_GEMM_CASE(6)
        BL_GEMM_CASE(7)
        BL_GEMM_CASE(8)
        BL_GEMM_CASE(9)
        default:
            return hipErrorInvalidValue;
    }
#undef BL_GEMM_CASE
}

}  // namespace bl
