// gemm32.hip -- prefill route of the ternary x int8 contraction on the
// 32 x 32 x 32 int8 MFMA (gfx950), for batches of 64 tokens and more.
//
// acc[m][n] = sum_k code(n, k) * q[m][k] - qsum[m], then optionally
// y[m][n] = (float)acc * (w_scale / inv[m]).
// [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU FFN":
// the prompt-processing GEMM over I2_S codes and int8 activations, which
// must write every output; codes offset by the activation sum.]
//
// Design.  A workgroup of WM x WN waves owns a BM x BN output tile (tokens
// x weight rows) and walks K one I2_S block (128 k) per step.  One block of
// one weight row is 32 bytes; the 16 bytes of half h hold, for each 2-bit
// field g, the codes of k = 32 g + 16 h + [0, 16) -- exactly what lane l of
// v_mfma_i32_32x32x32_i8 supplies for column l % 32 when h = l / 32.  So one
// 16-byte read per lane feeds the four MFMAs of a block (one per field),
// and the activation operand of field g is the 16 int8 q values at the same
// k.  (The hardware's order of k inside a lane never matters: both operands
// use the same lane/byte -> k map.)
//
// Both operands go global -> LDS by LDS-direct buffer loads (no register
// staging), into rings of distinct LDS objects: RA step buffers of
// activations (BM x 128 bytes) and RB >= RA of packed weights (BN x 32
// bytes), the weights running RB - RA steps further ahead since they come
// from HBM.  Per step a wave
//   1. waits for its own loads of the next step, then meets the workgroup
//      barrier (every wave's loads of the next step have landed, and every
//      wave is done reading the buffers the new loads will fill);
//   2. issues the loads of step t + RA (and weights of t + RB);
//   3. reads the next step's activation fragments and packed weights from
//      LDS into the other half of a register ping-pong, while
//   4. the MFMAs of the current step run over fragments read one step
//      earlier, the codes of field g + 1 expanded (shift + mask) in the
//      shadow of field g's MFMAs.
// So no MFMA waits for an LDS read issued in its own step, and RA - 1 steps
// of loads are in flight while one is contracted.  All loads are range-
// checked buffer loads (rows past M or N read zeros); K is a whole number of
// blocks on every path, so there is no K tail.
//
// k groups (KG = 2, with two blocks per step): the workgroup's waves form
// two groups of WM x WN, group g contracting block g of every step into its
// own accumulators, which group 1 hands to group 0 through LDS at the end.
// With the same tile and wave count, each wave then owns twice the output
// (64 x 64 instead of 64 x 32), so the fragments read from LDS per k fall
// by 44 %.
//
// LDS layouts (bank-conflict-free 16-byte reads of 16 lanes): activation
// row r (128 bytes, chunk c = 2 g + h) keeps chunk c at c ^ ((r >> 1) & 7);
// weight row r (32 bytes, half h) keeps half h at h ^ ((r >> 3) & 1).
#include <algorithm>
#include <climits>

#include "common.hpp"

namespace bl {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBlk = 128;  // k per step: one I2_S block

// D[32][32] += A[32][32] * B[32][32] (int8 -> int32).  Lane l supplies A
// row l % 32 and B column l % 32 (16 bytes each, k-group l / 32); D element
// (i, j) lives in lane j + 32 * ((i / 4) % 2), register 4 * (i / 8) + i % 4.
__device__ __forceinline__ v16i mfma32(const v4i &a, const v4i &b, const v16i &c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Explicit wait for this wave's vector-memory loads (at most VMCNT left),
// then the workgroup barrier (LDS traffic drained first).
template <int VMCNT>
__device__ __forceinline__ void wait_vm_barrier32() {
    static_assert(VMCNT >= 0 && VMCNT < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070 | (VMCNT & 15) | ((VMCNT >> 4) << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

constexpr int lcm_int(int a, int b) {
    int x = a, y = b;
    while (y) {
        const int t = x % y;
        x = y;
        y = t;
    }
    return a / x * b;
}

// Position of 16-byte chunk c of row r in a step buffer whose rows are
// 16 * NC bytes: an XOR swizzle that puts the same chunk of 16 consecutive
// rows on 16 distinct 4-bank groups (64 banks of 4 bytes).
template <int NC>
__device__ __forceinline__ int chunk_pos(int r, int c) {
    if constexpr (NC == 2) return c ^ ((r >> 3) & 1);
    else if constexpr (NC == 4) return c ^ ((r >> 2) & 3);
    else if constexpr (NC == 8) return c ^ ((r >> 1) & 7);
    else return c ^ (r & 15);
}

// One BM x BN output tile at (m0, n0) of one problem, by the whole
// workgroup, KB I2_S blocks per step.  YT: storage type of y (float,
// bf16_t, _Float16).
template <int BM, int BN, int WM, int WN, int KB, int RA, int RB, int KG, bool OUT_Y,
          typename YT>
__device__ __forceinline__ void gemm32_tile(const int8_t *__restrict__ q,
                                            const float *__restrict__ inv,
                                            const int32_t *__restrict__ qsum,
                                            const uint8_t *__restrict__ packed, float w_scale,
                                            int M, int K, int N, YT *__restrict__ y,
                                            int32_t *__restrict__ acc_out, int m0, int n0) {
    constexpr int NW = KG * WM * WN, NT = NW * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MI = TM / 32, NI = TN / 32;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile of whole 32 x 32 MFMA tiles");
    static_assert(KB == 1 || KB == 2, "blocks per step");
    static_assert(KG == 1 || KG == KB, "k groups: one block of each step per group");
    constexpr int BW = KB / KG;                // blocks of a step this wave contracts
    constexpr int NCA = 8 * KB, NCB = 2 * KB;  // 16-byte chunks per row of a step
    constexpr int NF = 4 * BW;                 // (block, field) pairs per step and wave
    // Bytes of one step (activations, packed weights), each rounded up to
    // whole loads of every lane: chunks past the step's data are loaded out
    // of range (zeros), so every wave issues the same number of loads.
    constexpr int SA = BM * 16 * NCA, SB = BN * 16 * NCB;
    constexpr int NDA = (SA + NT * 16 - 1) / (NT * 16), NDB = (SB + NT * 16 - 1) / (NT * 16);
    constexpr int SAP = NDA * NT * 16, SBP = NDB * NT * 16;
    static_assert(RA >= 2 && RB >= RA && RB <= 6 && RA <= 4, "ring depths");
    constexpr int UNROLL = lcm_int(lcm_int(2, RA), RB);
    static_assert(UNROLL <= 12, "unrolled ring");
    __shared__ __align__(16) int8_t a0[SAP], a1[SAP], a2[RA > 2 ? SAP : 16], a3[RA > 3 ? SAP : 16];
    __shared__ __align__(16) uint8_t b0[SBP], b1[SBP], b2[RB > 2 ? SBP : 16],
        b3[RB > 3 ? SBP : 16], b4[RB > 4 ? SBP : 16], b5[RB > 5 ? SBP : 16];
    __shared__ float sc_sh[BM];
    __shared__ int qs_sh[BM];
    auto ringA = [&](auto I) -> int8_t * {
        constexpr int i = decltype(I)::value % RA;
        if constexpr (i == 0) return a0;
        else if constexpr (i == 1) return a1;
        else if constexpr (i == 2) return a2;
        else return a3;
    };
    auto ringB = [&](auto I) -> uint8_t * {
        constexpr int i = decltype(I)::value % RB;
        if constexpr (i == 0) return b0;
        else if constexpr (i == 1) return b1;
        else if constexpr (i == 2) return b2;
        else if constexpr (i == 3) return b3;
        else if constexpr (i == 4) return b4;
        else return b5;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    // With KG > 1 the waves form KG groups of WM x WN, group kg contracting
    // block kg of every step into its own accumulators (summed at the end).
    const int kg = wid / (WM * WN), wt = wid % (WM * WN);
    const int wm = wt / WN, wn = wt % WN;
    const int l32 = lane & 31, hh = lane >> 5;
    const int nsteps = K / (kBlk * KB);
    const uint32_t rowbytes = (uint32_t)K / 4;
    const auto rq = make_rsrc(q + (size_t)m0 * K, (uint32_t)min(BM, M - m0) * (uint32_t)K);
    const auto rw = make_rsrc(packed + (size_t)n0 * rowbytes,
                              (uint32_t)min(BN, N - n0) * rowbytes);

    // Row scale and activation sum of the tile's rows, for the epilogue
    // (read before the loop; the barriers of the loop order them).
    for (int r = tid; r < BM; r += NT) {
        const int m = min(m0 + r, M - 1);
        qs_sh[r] = qsum[m];
        sc_sh[r] = OUT_Y ? w_scale / inv[m] : 0.0f;
    }

    // Source offsets of this lane's LDS-direct loads.  Load j of wave w
    // writes LDS chunk p = (j NW + w) 64 + lane; chunk c of a row is the
    // 16 bytes at k offset 16 c of the step (block c / 8 for activations,
    // c / 2 for packed weights).
    uint32_t asrc[NDA];
#pragma unroll
    for (int j = 0; j < NDA; ++j) {
        const int p = (j * NW + wid) * 64 + lane;
        const int row = p / NCA;
        const int c = chunk_pos<NCA>(row, p % NCA);  // the swizzle is an involution
        asrc[j] = p < SA / 16 ? (uint32_t)row * (uint32_t)K + 16u * (uint32_t)c : kOOB;
    }
    uint32_t bsrc[NDB];
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
        const int p = (j * NW + wid) * 64 + lane;
        const int row = p / NCB;
        const int c = chunk_pos<NCB>(row, p % NCB);
        bsrc[j] = p < SB / 16 ? (uint32_t)row * rowbytes + 16u * (uint32_t)c : kOOB;
    }
    // LDS offsets of this lane's fragment reads: activations of (block b,
    // field g) -- chunk 8 b + 2 g + half; packed weights of block b -- chunk
    // 2 b + half.
    int aoff[BW][4][MI];
#pragma unroll
    for (int b = 0; b < BW; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = wm * TM + 32 * mi + l32;
                aoff[b][g][mi] =
                    r * 16 * NCA + 16 * chunk_pos<NCA>(r, 8 * (kg * BW + b) + 2 * g + hh);
            }
    int boff[BW][NI];
#pragma unroll
    for (int b = 0; b < BW; ++b)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int r = wn * TN + 32 * ni + l32;
            boff[b][ni] = r * 16 * NCB + 16 * chunk_pos<NCB>(r, 2 * (kg * BW + b) + hh);
        }

    // Loads of step s: activations (A ring) and, RB - RA steps further on,
    // weights (B ring).  Steps past the end read zeros (the loads are still
    // issued, so every wave counts the same loads).
    auto issueA = [&](auto I, int s) {
        const uint32_t kb = (uint32_t)s * (kBlk * KB);
        const bool v = s < nsteps;
#pragma unroll
        for (int j = 0; j < NDA; ++j)
            buf_load16_lds(rq, ringA(I) + (j * NW + wid) * 1024, v ? asrc[j] : kOOB, kb);
    };
    auto issueB = [&](auto I, int s) {
        const uint32_t kb = (uint32_t)s * (32u * KB);
        const bool v = s < nsteps;
#pragma unroll
        for (int j = 0; j < NDB; ++j)
            buf_load16_lds(rw, ringB(I) + (j * NW + wid) * 1024, v ? bsrc[j] : kOOB, kb);
    };

    v16i acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0;

    v4i af[2][BW][4][MI];  // activation fragments, ping-pong by step parity
    v4i bp[2][BW][NI];     // packed weights, ping-pong by step parity
    v4i bx0[2][NI];        // expanded codes of block 0, field 0, by parity
    auto read_frags = [&](auto P, auto I) {
        constexpr int pp = decltype(P)::value;
        const uint8_t *bb = ringB(I);
#pragma unroll
        for (int b = 0; b < BW; ++b)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                bp[pp][b][ni] = *reinterpret_cast<const v4i *>(bb + boff[b][ni]);
        const int8_t *ab = ringA(I);
#pragma unroll
        for (int b = 0; b < BW; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    af[pp][b][g][mi] = *reinterpret_cast<const v4i *>(ab + aoff[b][g][mi]);
    };
    auto mfmas = [&](auto P, int b, int g, const v4i (&bf)[NI]) {
        constexpr int pp = decltype(P)::value;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                acc[mi][ni] = mfma32(af[pp][b][g][mi], bf[ni], acc[mi][ni]);
    };
    // MFMAs of (block, field) pairs 1 .. NF-1 of a step of parity pp (pair
    // 0 runs before the step's barrier); pair f + 1's codes are expanded
    // while pair f's MFMAs run, and block 0 / field 0 of the next step once
    // its packed weights have arrived.
    auto compute_rest = [&](auto P) {
        constexpr int pp = decltype(P)::value;
        v4i bf[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bf[ni] = unpack_field(bp[pp][0][ni], 1);
#pragma unroll
        for (int f = 1; f < NF; ++f) {
            v4i nb[NI];
            if (f + 1 < NF) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    nb[ni] = unpack_field(bp[pp][(f + 1) >> 2][ni], (f + 1) & 3);
            }
            mfmas(P, f >> 2, f & 3, bf);
            if (f + 1 < NF) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) bf[ni] = nb[ni];
            }
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bx0[pp ^ 1][ni] = unpack_field(bp[pp ^ 1][0][ni], 0);
    };

    // Prologue: the weights that run ahead, then RA groups (activations of
    // step s with weights of step s + RB - RA).
    constexpr int NG = NDA + NDB;  // loads per group
    unroll_ic([&](auto I) {
        constexpr int s = decltype(I)::value;
        if constexpr (s < RB - RA) issueB(ic<s>{}, s);
    }, std::make_integer_sequence<int, 6>{});
    unroll_ic([&](auto I) {
        constexpr int s = decltype(I)::value;
        if constexpr (s < RA) {
            issueA(ic<s>{}, s);
            issueB(ic<s + RB - RA>{}, s + RB - RA);
        }
    }, std::make_integer_sequence<int, 4>{});
    wait_vm_barrier32<(RA - 1) * NG>();
    read_frags(ic<0>{}, ic<0>{});
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bx0[0][ni] = unpack_field(bp[0][0][ni], 0);

    // Step t (ring position i = t mod UNROLL):
    //   the MFMAs of block 0 / field 0 (fragments and codes already in
    //   registers) go out first, so the matrix core works through the
    //   barrier;
    //   then the next step's loads have landed everywhere (wait + barrier)
    //   and the free buffers take step t + RA (weights t + RB);
    //   the next fragments are read while the rest of this step's MFMAs run.
    // The scheduler is told the order inside the second part (left to
    // itself it delays the next step's LDS reads until the current
    // fragments die, which exposes their latency at the next barrier): the
    // loads, the packed-weight reads, then the MFMAs one by one, each
    // followed by one fragment read while any are left and a few expansion
    // instructions.
    constexpr int NMF = (NF - 1) * MI * NI;     // MFMAs after the barrier
    constexpr int NRA = BW * 4 * MI;            // activation fragment reads
    constexpr int NVX = NI * (28 * BW);         // expansion instructions
    constexpr int VPER = (NVX + NMF - 1) / NMF;
    auto step = [&](auto I, int t) {
        constexpr int i = decltype(I)::value;
        constexpr int pp = i & 1;
        mfmas(ic<pp>{}, 0, 0, bx0[pp]);
        wait_vm_barrier32<(RA - 2) * NG>();
        issueA(ic<i + RA>{}, t + RA);
        issueB(ic<i + RB>{}, t + RB);
        read_frags(ic<pp ^ 1>{}, ic<i + 1>{});
        compute_rest(ic<pp>{});
        __builtin_amdgcn_sched_group_barrier(0x020, NG, 0);       // VMEM loads
        __builtin_amdgcn_sched_group_barrier(0x100, BW * NI, 0);  // packed-weight reads
        unroll_ic([&](auto Kk) {
            constexpr int k = decltype(Kk)::value;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if constexpr (k < NRA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);
        }, std::make_integer_sequence<int, NMF>{});
    };
    int t = 0;
    for (; t + UNROLL <= nsteps; t += UNROLL) {
        unroll_ic([&](auto I) { step(I, t + decltype(I)::value); },
                  std::make_integer_sequence<int, UNROLL>{});
    }
    // Remaining steps (fewer than UNROLL), same ring positions.
    unroll_ic([&](auto I) {
        if (t + decltype(I)::value < nsteps) step(I, t + decltype(I)::value);
    }, std::make_integer_sequence<int, UNROLL - 1>{});
    // Drain the trailing loads before the workgroup's LDS is released.
    wait_vm_barrier32<0>();

    if constexpr (KG == 2) {
        // Group 1 hands its accumulators to the group-0 wave of the same
        // (wm, wn) through the activation ring (free now): per wave MI x NI
        // x 16 ints a lane, 16-byte lane-contiguous chunks.
        static_assert(RA >= 2 && MI * NI * 4 * 1024 <= SAP, "hand-off space");
        int8_t *xa = wt < (WM * WN) / 2 ? a0 : a1;
        int8_t *xw = xa + (wt % ((WM * WN) / 2)) * (MI * NI * 4 * 1024);
        static_assert(((WM * WN) / 2) * MI * NI * 4 * 1024 <= SAP && (WM * WN) % 2 == 0,
                      "hand-off space per buffer");
        if (kg == 1) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const v4i v = {acc[mi][ni][4 * c], acc[mi][ni][4 * c + 1],
                                       acc[mi][ni][4 * c + 2], acc[mi][ni][4 * c + 3]};
                        *reinterpret_cast<v4i *>(xw + (((mi * NI + ni) * 4 + c) * 64 + lane) * 16) = v;
                    }
        }
        lds_barrier();
        if (kg == 1) return;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const v4i v = *reinterpret_cast<const v4i *>(
                        xw + (((mi * NI + ni) * 4 + c) * 64 + lane) * 16);
                    acc[mi][ni][4 * c] += v.x;
                    acc[mi][ni][4 * c + 1] += v.y;
                    acc[mi][ni][4 * c + 2] += v.z;
                    acc[mi][ni][4 * c + 3] += v.w;
                }
    }

    // Epilogue: D(i, j) of tile (mi, ni) in lane j + 32 ((i / 4) % 2),
    // register 4 (i / 8) + i % 4.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = wm * TM + 32 * mi + 8 * (e >> 2) + 4 * hh + (e & 3);
            const int m = m0 + r;
            if (m >= M) continue;
            const int qs = qs_sh[r];
            const float sc = sc_sh[r];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int n = n0 + wn * TN + 32 * ni + l32;
                if (n >= N) continue;
                const int v = acc[mi][ni][e] - qs;
                if constexpr (OUT_Y)
                    store_out(y, (size_t)m * N + n, (float)v * sc);
                else
                    acc_out[(size_t)m * N + n] = v;
            }
        }
    }
}

// Grouped form: up to 8 independent problems in one launch, every tile of
// every problem one workgroup (tiles of a problem ordered N-fastest).
struct G32Problem {
    const int8_t *q;
    const float *inv;
    const int32_t *qsum;
    const uint8_t *packed;
    void *y;
    int32_t *acc;
    float w_scale;
    int M, K, N;
    int tile_begin;  // first workgroup of this problem
    int ntn;         // tiles along N
};
constexpr int kMaxG32 = 8;
struct G32Batch {
    G32Problem p[kMaxG32];
};

// b0..b7: first workgroup of each problem (INT_MAX past the last), leading
// the argument list so that the build's kernel-argument preload puts them in
// scalar registers at wave launch.
// XCD: workgroups are dealt to the device's 8 chiplets (XCDs, each with its
// own L2) round-robin by index; with XCD set, workgroup b takes tile
// (b % 8) * ceil-share + b / 8, so each chiplet works through one
// contiguous run of tiles (the N tiles of a few row blocks) and its L2
// holds those rows' activations.
template <int BM, int BN, int WM, int WN, int KB, int RA, int RB, int KG, bool XCD, bool OUT_Y,
          typename YT>
__global__ __launch_bounds__(KG * WM * WN * 64) void gemm32_group_kernel(int b0, int b1, int b2, int b3,
                                                                    int b4, int b5, int b6, int b7,
                                                                    G32Batch B) {
    static_assert(kMaxG32 == 8, "one leading argument per problem");
    (void)b0;
    int bx = (int)blockIdx.x;
    if constexpr (XCD) {
        const int T = (int)gridDim.x, q8 = T >> 3, r8 = T & 7, x = bx & 7;
        bx = x * q8 + min(x, r8) + (bx >> 3);
    }
    const int pi = (bx >= b1) + (bx >= b2) + (bx >= b3) + (bx >= b4) + (bx >= b5) + (bx >= b6) +
                   (bx >= b7);
    const G32Batch *Bk = reinterpret_cast<const G32Batch *>(
        (const char *)__builtin_amdgcn_kernarg_segment_ptr() + 8 * sizeof(int));
    const G32Problem P = Bk->p[pi];
    const int t = bx - P.tile_begin;
    const int tm = t / P.ntn, tn = t - tm * P.ntn;
    gemm32_tile<BM, BN, WM, WN, KB, RA, RB, KG, OUT_Y, YT>(P.q, P.inv, P.qsum, P.packed, P.w_scale, P.M,
                                                    P.K, P.N, static_cast<YT *>(P.y), P.acc,
                                                    tm * BM, tn * BN);
}

struct Shape32 {
    int BM, BN, WM, WN, KB, RA, RB, KG;
    bool xcd;
};
// Launch-shape table; every entry computes bit-identical results.
constexpr Shape32 kShapes32[] = {
    {128, 128, 2, 2, 1, 3, 6, 1, false}, {128, 128, 2, 2, 2, 3, 6, 1, false},
    {128, 128, 2, 4, 1, 3, 3, 1, false}, {128, 128, 2, 4, 2, 3, 3, 1, false},
    {128, 128, 2, 2, 1, 3, 3, 1, false}, {128, 256, 2, 4, 1, 3, 6, 1, false},
    {128, 128, 2, 2, 2, 2, 4, 1, false}, {64, 128, 2, 2, 1, 3, 6, 1, false},
    {128, 128, 2, 2, 2, 3, 6, 1, true},  {128, 128, 2, 2, 1, 4, 4, 1, false},
    {128, 256, 2, 4, 1, 3, 6, 1, true},  {64, 128, 2, 2, 2, 3, 6, 1, false},
    {128, 128, 2, 2, 2, 3, 3, 2, false}};
constexpr int kNumShapes32 = sizeof(kShapes32) / sizeof(kShapes32[0]);

template <int BM, int BN, int WM, int WN, int KB, int RA, int RB, int KG, bool XCD>
hipError_t launch_g32(const GemmDesc *d, int count, hipStream_t s) {
    G32Batch B{};
    int begin[kMaxG32];
    int64_t total = 0;
    const bool y = d[0].y != nullptr;
    // Problems in order of decreasing K (stable): workgroups are dispatched
    // in index order, so the longest tiles start first and the short ones
    // fill in behind them, instead of the longest starting last (the
    // prefill layer's K = 6912 down projection behind six K = 2560 ones).
    int order[kMaxG32];
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order, order + count, [&](int a, int b) { return d[a].K > d[b].K; });
    for (int j = 0; j < count; ++j) {
        const int i = order[j];
        G32Problem &P = B.p[j];
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
    for (int i = count; i < kMaxG32; ++i) begin[i] = INT32_MAX;
    const dim3 grid((unsigned)total), block(KG * WM * WN * 64);
    const int io = d[0].io;
#define BL_G32(OY, YT)                                                                            \
    hipLaunchKernelGGL((gemm32_group_kernel<BM, BN, WM, WN, KB, RA, RB, KG, XCD, OY, YT>), grid,    \
                       block,                                                                     \
                       0,                                                                         \
                       s,                                                                        \
                       begin[0], begin[1], begin[2], begin[3], begin[4], begin[5], begin[6],     \
                       begin[7], B)
    if (y && io == kIoBf16)
        BL_G32(true, bf16_t);
    else if (y && io == kIoF16)
        BL_G32(true, _Float16);
    else if (y)
        BL_G32(true, float);
    else
        BL_G32(false, float);
#undef BL_G32
    return hipGetLastError();
}

}  // namespace

int gemm32_num_shapes() { return kNumShapes32; }

// Automatic shape: 128 x 128 tiles of 8 waves (two per SIMD, each 64 x 32),
// one block per step, 3-deep rings (72 KB of LDS: two workgroups per CU).
// Measured on MI355X against the 16 x 16 x 64 tile kernel: K = N = 8192 at
// M = 512 36.7 against 40 us, M = 2048 126 against 145-153 us; K = 2560,
// N = 6912 at M = 512 15.3 against 21 us.  With fewer than ~200 such tiles
// (N = 2560 at M = 512, or M = 256 at N = 8192) the smaller tiles of the
// 16 x 16 x 64 kernel fill the device better than these (for long rows the
// 64 x 128 shape below beats both).
constexpr int kAutoShape32 = 3;
// With >= 512 tiles of 128 x 256 (two per CU), the wider tile halves the
// activation traffic and wins (K = N = 8192 at M = 2048: 113-118 against
// 126-130 us); with >= 256 of them (one per CU) too when every row is long
// (K = N = 8192 at M = 1024: 53.1 against 59.6 us for the 128 x 128 tiles;
// the prefill layer's K = 2560 rows keep the narrower tile).
constexpr int kWideShape32 = 6;
// With at most one 128 x 128 tile per CU (every K a whole number of 256-k
// steps), the two k groups of 4 waves, each wave a 64 x 64 tile over its
// own block of every step: 44 % fewer LDS fragment reads per k than the
// 64 x 32 waves (K = N = 8192 at M = 512: 43-44.6 against 45-46.7 us per
// forward).  With more tiles its 121 KB of LDS (one workgroup per CU)
// loses to the 72 KB shape's two (prefill layer, 712 tiles: 74 against
// 68 us), and so it does on short rows, whose ten 256-k steps per tile do
// not amortise the two groups' hand-off (K = 2560, N = 6912 at M = 512:
// 15.4 against 14.4 us).
constexpr int kSplitShape32 = 13;
// 64 x 128 tiles, two blocks per step: for long rows at 64..255 tokens (or
// 256 with too few 128 x 128 tiles) whose 64 x 128 tiles number between
// three quarters of and one per CU.
constexpr int kHalfShape32 = 12;
constexpr int64_t kLongRowK = 4096;

// Shape the automatic choice takes for a set, or 0 where the 16 x 16 x 64
// kernel's tiles are taken.  Where every M >= 256 with >= 200 tiles of
// 128 x 128, the rules above.  Below that, long rows only (K >= 4096): the
// largest tile whose count lies between three quarters of and one per CU
// (128 x 256 and the two k groups of 128 x 128 from M = 96, 64 x 128 from
// M = 64), each measured against the 16 x 16 x 64 kernel's choice (tile
// kernel alone over q, K = 8192 unless given, us): M = 192, N = 28672
// 128 x 256 47.0 against 62.3; M = 96 / 128, N = 28672 split 30.2 / 31.7
// against 33.6 / 34.6; N = 8192 at M = 192 / 256 64 x 128 21.3 / 21.7
// against 23.5 / 23.8, K = 28672 at M = 192 59.3 against 62.2; M = 64,
// N = 28672 64 x 128 23.3 against 25.0 (the 128-row tiles, half empty,
// 28.4).  With more tiles than that (64 x 128 at M = 192, N = 28672: 60.7
// us) or fewer (M = 64, N = 16384: 21.7 against 17.5), the 16 x 16 x 64
// tiles stay.
int gemm32_auto_shape(const GemmDesc *d, int count) {
    int64_t wide = 0, tiles = 0, half = 0, mmin = INT64_MAX;
    bool even = true, long_rows = true;
    for (int i = 0; i < count; ++i) {
        wide += ((d[i].M + 127) / 128) * ((d[i].N + 255) / 256);
        tiles += ((d[i].M + 127) / 128) * ((d[i].N + 127) / 128);
        half += ((d[i].M + 63) / 64) * ((d[i].N + 127) / 128);
        mmin = std::min<int64_t>(mmin, d[i].M);
        even = even && d[i].K % (2 * kBlk) == 0;
        long_rows = long_rows && d[i].K >= kLongRowK;
    }
    const int64_t cus = device_cus(), most = 3 * cus / 4;
    if (mmin >= 256 && tiles >= 200)
        return (wide >= 2 * cus || (long_rows && wide >= cus)) ? kWideShape32
               : (even && long_rows && tiles <= cus)            ? kSplitShape32
                                                                : kAutoShape32;
    if (mmin < 64 || !long_rows) return 0;
    if (mmin >= 96 && wide >= most && wide <= cus) return kWideShape32;
    if (mmin >= 96 && even && tiles >= most && tiles <= cus) return kSplitShape32;
    if (even && half >= most && half <= cus) return kHalfShape32;
    return 0;
}

bool gemm32_preferred(const GemmDesc *d, int count) { return gemm32_auto_shape(d, count) != 0; }

hipError_t launch_gemm32_group(const GemmDesc *d, int count, int shape, hipStream_t s) {
    if (count < 1 || count > kMaxG32) return hipErrorInvalidValue;
    const bool y = d[0].y != nullptr;
    for (int i = 0; i < count; ++i)
        if (d[i].K % kBlk != 0 || (d[i].y != nullptr) != y || d[i].io != d[0].io)
            return hipErrorInvalidValue;
    int v = shape;
    if (v <= 0 || v > kNumShapes32) {
        v = gemm32_auto_shape(d, count);
        if (v == 0) v = kAutoShape32;
    }
    // Two blocks per step need an even block count in every row.
    if (kShapes32[v - 1].KB == 2)
        for (int i = 0; i < count; ++i)
            if (d[i].K % (2 * kBlk) != 0) v = 1;
#define BL_SHAPE32(idx)                                                                       \
    case idx:                                                                                 \
        return launch_g32<kShapes32[idx - 1].BM, kShapes32[idx - 1].BN, kShapes32[idx - 1].WM, \
                          kShapes32[idx - 1].WN, kShapes32[idx - 1].KB, kShapes32[idx - 1].RA, \
                          kShapes32[idx - 1].RB, kShapes32[idx - 1].KG,                       \
                          kShapes32[idx - 1].xcd>(d, count, s);
    switch (v) {
        BL_SHAPE32(1)
        BL_SHAPE32(2)
        BL_SHAPE32(3)
        BL_SHAPE32(4)
        BL_SHAPE32(5)
        BL_SHAPE32(6)
        BL_SHAPE32(7)
        BL_SHAPE32(8)
        BL_SHAPE32(9)
        BL_SHAPE32(10)
        BL_SHAPE32(11)
        BL_SHAPE32(12)
        BL_SHAPE32(13)
        default:
            return hipErrorInvalidValue;
    }
#undef BL_SHAPE32
}

}  // namespace bl
