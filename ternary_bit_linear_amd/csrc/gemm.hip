// gemm.hip -- prefill route of the ternary x int8 contraction (gfx950).
//
// acc[m][n] = sum_k code(n, k) * q[m][k] - qsum[m], then optionally
// y[m][n] = (float)acc * (w_scale / inv[m]).
// [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU FFN":
// the prompt-processing GEMM over I2_S codes and int8 activations, which
// must write every output; codes offset by the activation sum.]
//
// Design.  A workgroup of WM x WN waves owns a BM x BN output tile
// (tokens x weight rows) and walks K in 256-k steps (two I2_S blocks).  The
// int8 activations of a step go global -> LDS directly (LDS-direct buffer
// loads, no register staging) into a ring of R step buffers; the packed
// weights go global -> registers, one 16-byte load per lane per 16 weight
// rows (64 weights per lane), and are expanded there by shift+mask into
// the int8 B operand of v_mfma_i32_16x16x64_i8 (codes 0/1/2; the
// activation sum is subtracted in the epilogue).  R - 1 steps are in
// flight while one is contracted; one barrier per step.  Each wave keeps
// its (BM/WM) x (BN/WN) sub-tile in int32 accumulators.  All loads are
// range-checked buffer loads: ragged M, N and K tails read zeros.
#include <algorithm>
#include <climits>

#include "common.hpp"

namespace bl {
namespace {

// Ring-pipelined form.  The activation tile of each 256-k step is copied
// straight from global memory into LDS by buffer loads with the LDS-direct
// bit (lane i of a load writes bytes [16 i, 16 i + 16) after the wave's base
// address), into a ring of R step buffers: R - 1 steps are in flight while
// one is contracted.  The packed weights of a step go to registers, in a
// ring of R slots advanced with the LDS ring.
//
// In a step buffer a row is 256 bytes and its 16-byte chunk c sits at
// position (c + 2 (row % 8)) % 16, which puts the 16 rows x 4 k-groups of an
// MFMA fragment read on distinct LDS banks (the bank pattern of rows padded
// to 288 bytes, without the padding).
//
// The loop runs whole turns of the ring only (R is picked to divide the step
// count where possible; otherwise the last turn runs past K on loads that
// read zeros), so it has no early exit: every load issued is consumed on
// every path, the compiler can neither sink nor drop one, and the explicit
// waits can count loads exactly.  The step buffers are distinct LDS objects
// so that the compiler's own LDS-DMA wait tracking can tell them apart.
template <int VMCNT>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(VMCNT >= 0 && VMCNT < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070 | (VMCNT & 15) | ((VMCNT >> 4) << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One BM x BN output tile at (m0, n0) of one problem, by the whole
// workgroup.
// YT: storage type of y (float, bf16_t, _Float16; rounded to nearest even).
// WK: k groups.  With WK > 1 the workgroup holds WK groups of WM x WN
// waves; group g walks its own contiguous run of ceil(steps / WK) steps
// through a ring of its own, and the groups' int32 partial tiles are added
// in LDS at the end (integer sums: the result does not depend on WK).  This
// multiplies the loads in flight per tile, for grids of few tiles over long
// rows.
template <int BM, int BN, int WM, int WN, int R, bool KTAIL, bool OUT_Y, typename YT = float,
          int WK = 1>
__device__ __forceinline__ void gemm_tile(
    const int8_t *__restrict__ q, const float *__restrict__ inv,
    const int32_t *__restrict__ qsum, const uint8_t *__restrict__ packed,
    float w_scale, int M, int K, int N, YT *__restrict__ y,
    int32_t *__restrict__ acc_out, int m0, int n0) {
    constexpr int NW = WM * WN, NT = NW * 64;  // waves and threads of one k group
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MI = TM / 16, NI = TN / 16;
    constexpr int SB = BM * kStepK;            // activation bytes of one step
    constexpr int ND = SB / (NT * 16);         // LDS-direct loads per lane per step
    constexpr int GB = SB * WK;                // one ring slot of every k group
    static_assert(SB % (NT * 16) == 0, "step tile splits into whole wave loads");
    static_assert(R >= 3 && R <= 5 && R * GB <= 160 * 1024, "ring depth");
    static_assert(WK >= 1 && NW * WK <= 16, "at most 16 waves");
    __shared__ __align__(16) int8_t l0[GB], l1[GB], l2[GB], l3[R > 3 ? GB : 16],
        l4[R > 4 ? GB : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave-uniform (keeps derived resources scalar): k group and wave in it.
    const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kgi = WK > 1 ? wall / NW : 0;
    const int wid = WK > 1 ? wall - kgi * NW : wall;
    const int kgo = kgi * SB;
    auto ring = [&](auto I) -> int8_t * {
        constexpr int i = decltype(I)::value % R;
        if constexpr (i == 0) return l0 + kgo;
        else if constexpr (i == 1) return l1 + kgo;
        else if constexpr (i == 2) return l2 + kgo;
        else if constexpr (i == 3) return l3 + kgo;
        else return l4 + kgo;
    };
    const int wm = wid / WN, wn = wid % WN;
    const int j = lane & 15, kg = lane >> 4;
    const int nsteps = (K + kStepK - 1) / kStepK;
    const int spg = WK > 1 ? (nsteps + WK - 1) / WK : nsteps;  // steps of one k group
    const int sg0 = kgi * spg;                                  // its first step
    const int nblocks = K / kBlockWeights;
    const uint32_t rowbytes = (uint32_t)K / 4;
    const auto rq = make_rsrc(q + (size_t)m0 * K, (uint32_t)min(BM, M - m0) * (uint32_t)K);
    const auto rw = make_rsrc(packed + (size_t)n0 * rowbytes,
                              (uint32_t)min(BN, N - n0) * rowbytes);

    // Source of each of this lane's LDS-direct loads: position
    // p = (c NW + wave) 64 + lane holds row p / 16, chunk (p % 16 - 2 row) % 16.
    uint32_t dsrc[ND];
    int dk[ND];
#pragma unroll
    for (int c = 0; c < ND; ++c) {
        const int p = (c * NW + wid) * 64 + lane;
        const int row = p >> 4;
        const int ch = ((p & 15) - 2 * (row & 7)) & 15;
        dsrc[c] = (uint32_t)row * (uint32_t)K + 16u * ch;
        dk[c] = 16 * ch;
    }
    // LDS byte offsets of this lane's fragment of field g (row j, logical
    // chunk 8 (kg / 2) + kg % 2 + 2 g).
    int aoff[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int ch = 8 * (kg >> 1) + (kg & 1) + 2 * g;
        aoff[g] = (wm * TM + j) * kStepK + 16 * ((ch + 2 * (j & 7)) & 15);
    }
    // Per-lane weight offsets (row, k-group) of this wave's 16-row groups.
    uint32_t boff[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
        boff[ni] = (uint32_t)(wn * TN + 16 * ni + j) * rowbytes + 16u * kg;

    // Loads of the group's step sl, activations then weights.  When K is a
    // whole number of steps (KTAIL false) the step's k offset rides in the
    // scalar offset and steps past the end (of K, or of the group's run) are
    // redirected out of range (they read zeros); otherwise each chunk past K
    // is.
    auto issue = [&](int8_t *buf, v4i(&breg)[NI], int sl) {
        const int s = sg0 + sl;
        const bool run = WK == 1 || sl < spg;  // wave-uniform
        const int kb = s * kStepK;
#pragma unroll
        for (int c = 0; c < ND; ++c) {
            uint32_t off, soff;
            if constexpr (!KTAIL) {
                off = run && s < nsteps ? dsrc[c] : kOOB;
                soff = WK == 1 || run ? kb : 0;
            } else {
                off = run && kb + dk[c] < K ? dsrc[c] + (uint32_t)kb : kOOB;
                soff = 0;
            }
            buf_load16_lds(rq, buf + (c * NW + wid) * 1024, off, soff);
        }
        const bool kv = run && (KTAIL ? 2 * s + (kg >> 1) < nblocks : s < nsteps);
        const uint32_t wso = WK == 1 || run ? (uint32_t)s * kStepBytes : 0u;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) breg[ni] = buf_load16_so(rw, kv ? boff[ni] : kOOB, wso);
    };

    v4i acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4i{0, 0, 0, 0};

    // One step: the A fragments are read from LDS up front; then the MFMAs
    // of field g are interleaved with the expansion of field g + 1's B codes
    // (one MFMA, then two VALU instructions), so the vector ALU works in the
    // shadow of the matrix core.
    auto compute = [&](const int8_t *buf, const v4i(&breg)[NI]) {
        v4i a[4][MI];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                a[g][mi] = *reinterpret_cast<const v4i *>(buf + aoff[g] + 16 * mi * kStepK);
        v4i bf[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bf[ni] = unpack_field(breg[ni], 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            v4i nb[NI];
            if (g < 3) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) nb[ni] = unpack_field(breg[ni], g + 1);
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma16(a[g][mi], bf[ni], acc[mi][ni]);
#pragma unroll
            for (int k = 0; k < MI * NI; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
            if (g < 3) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) bf[ni] = nb[ni];
            }
        }
    };

    // Steps 0..R-2 are issued up front and step t + R - 1 at the top of
    // step t, into the buffer and slot step t - 1 used.  At the top of step
    // t its own loads must have landed; only steps t + 1 .. t + R - 2 may
    // still be in flight.
    constexpr int kPend = (R - 2) * (ND + NI);
    v4i breg[R][NI];
    unroll_ic([&](auto I) {
        if constexpr (decltype(I)::value < R - 1) {
            issue(ring(I), breg[decltype(I)::value], decltype(I)::value);
            __builtin_amdgcn_sched_barrier(0);
        }
    }, std::make_integer_sequence<int, R>{});
    const int turns = (spg + R - 1) / R;
    int s = 0;
    for (int t = 0; t < turns; ++t, s += R) {
        unroll_ic([&](auto I) {
            constexpr int i = decltype(I)::value;
            wait_vm_barrier<kPend>();
            issue(ring(ic<i + R - 1>{}), breg[(i + R - 1) % R], s + i + R - 1);
            __builtin_amdgcn_sched_barrier(0);
            compute(ring(I), breg[i]);
        }, std::make_integer_sequence<int, R>{});
    }
    // Drain the trailing loads before the workgroup's LDS is released.
    wait_vm_barrier<0>();

    if constexpr (WK > 1) {
        // Groups 1..WK-1 leave their partial tiles in the (now idle) first
        // ring slot; group 0 adds them in group order and writes the tile.
        static_assert((WK - 1) * NW * MI * NI * 64 * 16 <= GB, "partials fit one ring slot");
        v4i *part = reinterpret_cast<v4i *>(l0);
        auto at = [&](int g, int mi, int ni) {
            return (((g - 1) * NW + wid) * MI * NI + mi * NI + ni) * 64 + lane;
        };
        if (kgi > 0) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) part[at(kgi, mi, ni)] = acc[mi][ni];
        }
        __syncthreads();
        if (kgi > 0) return;
#pragma unroll
        for (int g = 1; g < WK; ++g)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) acc[mi][ni] += part[at(g, mi, ni)];
    }

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
                    store_out(y, (size_t)m * N + n, (float)v * sc);
                else
                    acc_out[(size_t)m * N + n] = v;
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int R, bool KTAIL, bool OUT_Y, int WK>
__global__ __launch_bounds__(WM * WN * WK * 64) void gemm_ring_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ inv,
    const int32_t *__restrict__ qsum, const uint8_t *__restrict__ packed,
    float w_scale, int M, int K, int N, float *__restrict__ y,
    int32_t *__restrict__ acc_out) {
    gemm_tile<BM, BN, WM, WN, R, KTAIL, OUT_Y, float, WK>(
        q, inv, qsum, packed, w_scale, M, K, N, y, acc_out, (int)blockIdx.y * BM,
        (int)blockIdx.x * BN);
}

// Grouped form: up to 8 independent problems (K a whole number of steps)
// in one launch, every tile of every problem one workgroup.
struct GroupProblem {
    const int8_t *q;
    const float *inv;
    const int32_t *qsum;
    const uint8_t *packed;
    float *y;
    int32_t *acc;
    float w_scale;
    int M, K, N;
    int tile_begin;  // first workgroup of this problem
    int ntn;         // tiles along N
};
constexpr int kMaxGroup = 8;
struct GroupBatch {
    GroupProblem p[kMaxGroup];
};

// b0..b7: first workgroup of each problem (INT_MAX past the last); they
// lead the argument list so that the build's kernel-argument preload puts
// them in scalar registers at wave launch.  Tiles of a problem are ordered
// N-fastest, as in the single-problem grid.
template <int BM, int BN, int WM, int WN, int R, bool OUT_Y, typename YT, int WK>
__global__ __launch_bounds__(WM * WN * WK * 64) void gemm_group_kernel(int b0, int b1, int b2, int b3,
                                                                  int b4, int b5, int b6, int b7,
                                                                  GroupBatch B) {
    static_assert(kMaxGroup == 8, "one leading argument per problem");
    (void)b0;
    const int bx = (int)blockIdx.x;
    const int pi = (bx >= b1) + (bx >= b2) + (bx >= b3) + (bx >= b4) + (bx >= b5) + (bx >= b6) +
                   (bx >= b7);
    const GroupBatch *Bk = reinterpret_cast<const GroupBatch *>(
        (const char *)__builtin_amdgcn_kernarg_segment_ptr() + 8 * sizeof(int));
    const GroupProblem P = Bk->p[pi];
    const int t = bx - P.tile_begin;
    const int tm = t / P.ntn, tn = t - tm * P.ntn;
    gemm_tile<BM, BN, WM, WN, R, false, OUT_Y, YT, WK>(P.q, P.inv, P.qsum, P.packed, P.w_scale,
                                                       P.M, P.K, P.N, reinterpret_cast<YT *>(P.y),
                                                       P.acc, tm * BM, tn * BN);
}

struct Tile {
    int BM, BN, WM, WN, R;  // R == 0: ring depth picked from the step count
    int WK = 1;             // k groups
};
// Launch-shape table; every entry computes bit-identical results.
constexpr Tile kTiles[] = {{64, 256, 1, 4, 3}, {64, 128, 1, 4, 3}, {64, 64, 2, 2, 0},
                           {32, 64, 1, 4, 0},  {32, 128, 1, 4, 0}, {128, 128, 1, 4, 3},
                           {128, 256, 1, 4, 3}, {64, 256, 1, 4, 4}, {64, 128, 1, 4, 0},
                           {128, 128, 2, 2, 0}, {64, 64, 2, 2, 3},  {32, 64, 1, 4, 3},
                           {128, 256, 2, 4, 3}, {64, 512, 1, 8, 3}, {64, 512, 1, 8, 4},
                           {64, 512, 1, 8, 5},  {64, 256, 1, 8, 4}, {32, 512, 1, 8, 4},
                           {16, 256, 1, 4, 0},  {16, 128, 1, 4, 0}, {32, 32, 2, 2, 0},
                           {16, 32, 1, 2, 0},   {16, 64, 1, 4, 0},  {16, 32, 1, 2, 0, 2},
                           {16, 32, 1, 2, 0, 4}, {16, 32, 1, 2, 0, 8}, {16, 64, 1, 4, 0, 2},
                           {16, 64, 1, 4, 0, 4}, {16, 128, 1, 4, 0, 2}, {16, 16, 1, 1, 0, 4},
                           {16, 16, 1, 1, 0, 8}, {32, 64, 1, 4, 0, 2}, {32, 64, 1, 4, 0, 4},
                           {64, 128, 1, 4, 0, 2}, {32, 128, 1, 4, 0, 2}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
static_assert(kNumTiles == 35, "one BL_GEMM_CASE per table entry");

// Ring depth for a tile: the deepest of 4, 5, 3 that divides the step count
// of one k group (no padded steps), else 4.  Depths whose ring does not fit
// the LDS are skipped.
int pick_depth(int bm, int64_t K, int wk = 1) {
    const int64_t nsteps = ((K + kStepK - 1) / kStepK + wk - 1) / wk;
    for (int r : {4, 5, 3})
        if ((int64_t)r * bm * kStepK * wk <= 160 * 1024 && nsteps % r == 0) return r;
    return 4;
}

template <int BM, int BN, int WM, int WN, int R, int WK = 1>
hipError_t launch_ring(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M, int64_t K, int64_t N,
                       float *y, int32_t *acc, hipStream_t s) {
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    const dim3 block(WM * WN * WK * 64);
    const bool kt = K % kStepK != 0;
#define BL_RING_LAUNCH(KT, OY)                                                                  \
    hipLaunchKernelGGL((gemm_ring_kernel<BM, BN, WM, WN, R, KT, OY, WK>), grid, block, 0, s, q, \
                       inv, qsum, packed, w_scale, (int)M, (int)K, (int)N, y, acc)
    if (y) {
        if (kt)
            BL_RING_LAUNCH(true, true);
        else
            BL_RING_LAUNCH(false, true);
    } else {
        if (kt)
            BL_RING_LAUNCH(true, false);
        else
            BL_RING_LAUNCH(false, false);
    }
#undef BL_RING_LAUNCH
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int RFIX, int WK>
hipError_t launch_tile(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M, int64_t K, int64_t N,
                       float *y, int32_t *acc, hipStream_t s) {
    if constexpr (RFIX != 0) {
        return launch_ring<BM, BN, WM, WN, RFIX, WK>(q, inv, qsum, packed, w_scale, M, K, N, y,
                                                     acc, s);
    } else {
        const int r = pick_depth(BM, K, WK);
        if (r == 3)
            return launch_ring<BM, BN, WM, WN, 3, WK>(q, inv, qsum, packed, w_scale, M, K, N, y,
                                                      acc, s);
        if constexpr (5 * BM * kStepK * WK <= 160 * 1024)
            if (r == 5)
                return launch_ring<BM, BN, WM, WN, 5, WK>(q, inv, qsum, packed, w_scale, M, K, N,
                                                          y, acc, s);
        return launch_ring<BM, BN, WM, WN, 4, WK>(q, inv, qsum, packed, w_scale, M, K, N, y, acc,
                                                  s);
    }
}

}  // namespace

int gemm_num_variants() { return kNumTiles + gemm32_num_shapes(); }

bool gemm_group_supported(int64_t K) { return K % kStepK == 0; }

namespace {

template <int BM, int BN, int WM, int WN, int R, int WK = 1>
hipError_t launch_group_tile(const GemmDesc *d, int count, hipStream_t s) {
    GroupBatch B{};
    int begin[kMaxGroup];
    int64_t total = 0;
    const bool y = d[0].y != nullptr;
    // Problems in order of decreasing K (stable): the longest tiles are
    // dispatched first, the short ones fill in behind them.
    int order[kMaxGroup];
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order, order + count, [&](int a, int b) { return d[a].K > d[b].K; });
    for (int j = 0; j < count; ++j) {
        const int i = order[j];
        GroupProblem &P = B.p[j];
        P.q = d[i].q;
        P.inv = d[i].inv;
        P.qsum = d[i].qsum;
        P.packed = d[i].packed;
        P.y = d[i].y;
        P.acc = d[i].acc;
        P.w_scale = d[i].w_scale;
        P.M = (int)d[i].M;
        P.K = (int)d[i].K;
        P.N = (int)d[i].N;
        const int64_t ntn = (d[i].N + BN - 1) / BN, ntm = (d[i].M + BM - 1) / BM;
        P.ntn = (int)ntn;
        P.tile_begin = (int)total;
        begin[j] = (int)total;
        total += ntn * ntm;
        if (total > INT32_MAX) return hipErrorInvalidConfiguration;
    }
    for (int i = count; i < kMaxGroup; ++i) begin[i] = INT32_MAX;
    const dim3 grid((unsigned)total), block(WM * WN * WK * 64);
    const int io = d[0].io;
    if (y && io == kIoBf16)
        hipLaunchKernelGGL((gemm_group_kernel<BM, BN, WM, WN, R, true, bf16_t, WK>), grid, block, 0,
                           s, begin[0], begin[1], begin[2], begin[3], begin[4], begin[5], begin[6],
                           begin[7], B);
    else if (y && io == kIoF16)
        hipLaunchKernelGGL((gemm_group_kernel<BM, BN, WM, WN, R, true, _Float16, WK>), grid, block,
                           0, s, begin[0], begin[1], begin[2], begin[3], begin[4], begin[5],
                           begin[6], begin[7], B);
    else if (y)
        hipLaunchKernelGGL((gemm_group_kernel<BM, BN, WM, WN, R, true, float, WK>), grid, block, 0,
                           s, begin[0], begin[1], begin[2], begin[3], begin[4], begin[5], begin[6],
                           begin[7], B);
    else
        hipLaunchKernelGGL((gemm_group_kernel<BM, BN, WM, WN, R, false, float, WK>), grid, block, 0,
                           s, begin[0], begin[1], begin[2], begin[3], begin[4], begin[5], begin[6],
                           begin[7], B);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_group(const GemmDesc *d, int count, hipStream_t s) {
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
    if (gemm32_preferred(d, count)) return launch_gemm32_group(d, count, 0, s);
    const bool y = d[0].y != nullptr;
    int64_t t64x512 = 0, t64x256 = 0, t64x128 = 0, t32x128 = 0, t16x128 = 0, t16x64 = 0, kmax = 0,
            mmax = 0;
    double work = 0.0, work_k = 0.0;  // int ops, and int ops x K
    for (int i = 0; i < count; ++i) {
        if (!gemm_group_supported(d[i].K) || (d[i].y != nullptr) != y || d[i].io != d[0].io)
            return hipErrorInvalidValue;
        auto tiles = [&](int bm, int bn) {
            return ((d[i].M + bm - 1) / bm) * ((d[i].N + bn - 1) / bn);
        };
        t64x512 += tiles(64, 512);
        t64x256 += tiles(64, 256);
        t64x128 += tiles(64, 128);
        t32x128 += tiles(32, 128);
        t16x128 += tiles(16, 128);
        t16x64 += tiles(16, 64);
        kmax = std::max<int64_t>(kmax, d[i].K);
        mmax = std::max<int64_t>(mmax, d[i].M);
        const double w = (double)d[i].M * (double)d[i].N * (double)d[i].K;
        work += w;
        work_k += w * (double)d[i].K;
    }
    const double k_avg = work_k / work;  // K of the average int op
    // The single-problem rule (launch_gemm) applied to the group's tile
    // counts; one ring depth for all problems (steps past a problem's K
    // read zeros).
    // Ring depth (4 or 5) with the fewest padded steps, weighted by work: a
    // problem's last ring turn runs past its K on loads that read zeros.
    double pad4 = 0.0, pad5 = 0.0;
    for (int i = 0; i < count; ++i) {
        const double w = (double)d[i].M * (double)d[i].N * (double)d[i].K;
        const int64_t ns = d[i].K / kStepK;
        pad4 += w * (double)((4 - ns % 4) % 4) / (double)ns;
        pad5 += w * (double)((5 - ns % 5) % 5) / (double)ns;
    }
    const bool r5 = pad5 < pad4;
    if (mmax <= 32) {
        // Few tokens: 16-row tiles, as for a single problem (the 16x32 tiles
        // in 4 k groups, their ring depth from the steps of one group).
        if (t16x128 >= 200)
            return r5 ? launch_group_tile<16, 128, 1, 4, 5>(d, count, s)
                      : launch_group_tile<16, 128, 1, 4, 4>(d, count, s);
        if (t16x64 >= 200)
            return r5 ? launch_group_tile<16, 64, 1, 4, 5>(d, count, s)
                      : launch_group_tile<16, 64, 1, 4, 4>(d, count, s);
        double g4 = 0.0, g5 = 0.0;
        for (int i = 0; i < count; ++i) {
            const double w = (double)d[i].M * (double)d[i].N * (double)d[i].K;
            const int64_t ns = (d[i].K / kStepK + 3) / 4;
            g4 += w * (double)((4 - ns % 4) % 4) / (double)ns;
            g5 += w * (double)((5 - ns % 5) % 5) / (double)ns;
        }
        return g5 < g4 ? launch_group_tile<16, 32, 1, 2, 5, 4>(d, count, s)
                       : launch_group_tile<16, 32, 1, 2, 4, 4>(d, count, s);
    }
    // The 64-row tiles from three quarters of a tile per CU (M = 64..128 at
    // N = 28672, K = 8192: 64x128 over 32x128 at M = 64, 28.9 -> 25.1 us;
    // 64x256 over 64x128 at M = 96 / 128, 35.7 -> 33.5 / 37.8 -> 34.9 us;
    // M = 192, K = N = 8192: 64x128 over 32x128, 24.2 -> 23.6 us).
    const int64_t most = 3 * (int64_t)device_cus() / 4;
    if (t64x512 >= 512) return launch_group_tile<64, 512, 1, 8, 4>(d, count, s);
    if (k_avg >= 6144.0 && t64x256 >= most) return launch_group_tile<64, 256, 1, 8, 4>(d, count, s);
    if (t64x128 >= most)
        // Short rows (a few ring turns per tile): a 3-deep ring, so that two
        // workgroups share a CU and one's fill hides behind the other's
        // MFMAs (decoder layer at M = 512, K mostly 2560: 82 -> 75 us).
        return k_avg <= 4096.0 ? launch_group_tile<64, 128, 1, 4, 3>(d, count, s)
               : r5            ? launch_group_tile<64, 128, 1, 4, 5>(d, count, s)
                               : launch_group_tile<64, 128, 1, 4, 4>(d, count, s);
    if (kmax > 4096 && t32x128 >= 256)
        return r5 ? launch_group_tile<32, 128, 1, 4, 5>(d, count, s)
                  : launch_group_tile<32, 128, 1, 4, 4>(d, count, s);
    return r5 ? launch_group_tile<32, 64, 1, 4, 5>(d, count, s)
              : launch_group_tile<32, 64, 1, 4, 4>(d, count, s);
}

hipError_t launch_gemm(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, int64_t N, float *y, int32_t *acc,
                       int variant, hipStream_t s) {
    int v = variant;
    if (v <= 0) {
        // Picked from a sweep on MI355X: the widest tiles (8 waves, a 4-step
        // ring) when the grid still has two workgroups per CU, then 64x256
        // (8 waves; long K only: short rows do not amortise its fill), 64x128
        // down to one per CU, then 32-row tiles (the wider one for long K).
        auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
        const GemmDesc one{q, inv, qsum, packed, w_scale, M, K, N, y, acc};
        if (gemm32_preferred(&one, 1)) {
            return launch_gemm32_group(&one, 1, 0, s);
        } else if (M <= 32)
            // Few tokens: 16-row tiles, the widest that still gives about one
            // tile per CU (M = 16, K = 8192: N = 8192 16x32 8.8 us against
            // 32x64 10.3 us; N = 28672 16x128; measured).  The 16x32 tiles
            // run in 4 k groups: 2 waves per tile keep too few loads in
            // flight (M = 16, N = 8192: K = 8192 8.8 -> 7.2 us, K = 28672
            // 25.7 -> 18.4 us; K = 2560 level).  The wider tiles gained
            // nothing from k groups.
            v = tiles(16, 128) >= 200 ? 20 : tiles(16, 64) >= 200 ? 23 : 25;
        else if (tiles(64, 512) >= 512)
            v = 15;
        // The 64-row tiles from three quarters of a tile per CU, as in the
        // grouped launch.  Past 16384-long rows the 32-row tiles run in k
        // groups (K = 28672, N = 8192: M = 64 32x64 33.4 -> 31.1 us, M = 128
        // 32x128 48.4 -> 45.6 us; at K = 8192 level or slower).
        else if (K >= 6144 && tiles(64, 256) >= 3 * (int64_t)device_cus() / 4)
            v = 17;
        else if (tiles(64, 128) >= 3 * (int64_t)device_cus() / 4)
            v = 9;
        else if (K > 4096 && tiles(32, 128) >= 256)
            v = K >= 16384 ? 35 : 5;
        else
            v = K >= 16384 ? 32 : 4;
    }
    if (v > kNumTiles) {
        // Variants past the 16 x 16 x 64 table: the 32 x 32 x 32 kernel's
        // launch shapes (K % 128 == 0 always holds here).
        GemmDesc d{q, inv, qsum, packed, w_scale, M, K, N, y, acc};
        return launch_gemm32_group(&d, 1, v - kNumTiles, s);
    }
#define BL_GEMM_CASE(idx)                                                                  \
    case idx:                                                                              \
        return launch_tile<kTiles[idx - 1].BM, kTiles[idx - 1].BN, kTiles[idx - 1].WM,     \
                           kTiles[idx - 1].WN, kTiles[idx - 1].R, kTiles[idx - 1].WK>(       \
            q, inv, qsum, packed, w_scale, M, K, N, y, acc, s);
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
        BL_GEMM_CASE(10)
        BL_GEMM_CASE(11)
        BL_GEMM_CASE(12)
        BL_GEMM_CASE(13)
        BL_GEMM_CASE(14)
        BL_GEMM_CASE(15)
        BL_GEMM_CASE(16)
        BL_GEMM_CASE(17)
        BL_GEMM_CASE(18)
        BL_GEMM_CASE(19)
        BL_GEMM_CASE(20)
        BL_GEMM_CASE(21)
        BL_GEMM_CASE(22)
        BL_GEMM_CASE(23)
        BL_GEMM_CASE(24)
        BL_GEMM_CASE(25)
        BL_GEMM_CASE(26)
        BL_GEMM_CASE(27)
        BL_GEMM_CASE(28)
        BL_GEMM_CASE(29)
        BL_GEMM_CASE(30)
        BL_GEMM_CASE(31)
        BL_GEMM_CASE(32)
        BL_GEMM_CASE(33)
        BL_GEMM_CASE(34)
        BL_GEMM_CASE(35)
        default:
            return hipErrorInvalidValue;
    }
#undef BL_GEMM_CASE
}

}  // namespace bl
