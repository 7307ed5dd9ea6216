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
#include <algorithm>

#include "common.hpp"

namespace bl {
namespace {

constexpr int kW = 4;           // waves per workgroup
constexpr int kTileRows = 8;    // weight rows per tile
constexpr int kStep = 128;      // packed bytes of a row per step (512 k)

struct LdsRowSink {
    static constexpr bool kDeferSum = false;
    int8_t *q;
    float *inv;
    int *qsum;
    __device__ void store_q(int k, uint32_t v) { *reinterpret_cast<uint32_t *>(q + k) = v; }
    __device__ void store_row(float iv, int qs) {
        *inv = iv;
        *qsum = qs;
    }
};

// Arguments of one contraction (one BitLinear) as seen by a workgroup.
// The 4 waves of a workgroup work on 4 / ks tile groups at once (a set),
// ks waves splitting each tile group's K range.  tg_first / tg_stride:
// this workgroup's first set and the stride of its walk (its index and the
// number of workgroups on this problem).
struct GemvArgs {
    const float *x;
    const float *gamma;
    const int8_t *q;
    const float *inv;
    const int32_t *qsum;
    const uint8_t *packed;
    float *y;
    int32_t *acc_out;
    int8_t *q_out;
    float *inv_out;
    int32_t *qsum_out;
    float eps;
    float w_scale;
    int M, K, N;
    int m0;
    int tg_first, tg_stride;  // in units of tile-group sets (see ks)
    int ks;                   // waves per tile group (K split): 1, 2 or 4
};

// Decode contraction of one workgroup.  FM (MODE 0): compile-time bound on
// the token rows (M <= FM); LONG (MODE 0): rows longer than 8192 take the
// streamed normalisation.  TH: token halves (1 for M <= 8, 2 for M <= 16).
template <int R, int U, int MODE, bool OUT_Y, int FM, bool LONG, int TH>
__device__ __forceinline__ void gemv_body(const GemvArgs &A) {
    extern __shared__ __align__(16) int8_t q_lds[];
    const float *__restrict__ x = A.x;
    const float *__restrict__ gamma = A.gamma;
    const int8_t *__restrict__ q = A.q;
    const float *__restrict__ inv = A.inv;
    const int32_t *__restrict__ qsum = A.qsum;
    const uint8_t *__restrict__ packed = A.packed;
    float *__restrict__ y = A.y;
    int32_t *__restrict__ acc_out = A.acc_out;
    const float eps = A.eps, w_scale = A.w_scale;
    const int M = A.M, K = A.K, N = A.N;
    __shared__ float red[kRedWords];
    __shared__ float inv_sh[4];
    __shared__ int qsum_sh[4];
    __shared__ v4i part[kW][TH][R][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps derived resources scalar
    const int r8 = lane & 7;    // weight row within the tile (load role)
    const int ch = lane >> 3;   // 16-byte chunk within the 128-byte step
    const int m0 = A.m0;
    const int mg = min(16, M - m0);  // tokens of this workgroup's group

    const uint32_t rowbytes = (uint32_t)K / 4;
    const int nsteps = (int)((rowbytes + kStep - 1) / kStep);
    const int ks = A.ks;
    const int slots = kW / ks;                // tile groups per set
    const int sg = wid / ks, kp = wid % ks;   // this wave's tile group slot / K part
    const int nb = (nsteps + ks * U - 1) / (ks * U);
    const int ntg = (N + kTileRows * R - 1) / (kTileRows * R);
    const int nset = (ntg + slots - 1) / slots;
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

    int st = A.tg_first;  // current set
    int b = 0;

    // Weights of batch b_ of this wave's tile group in set st_ (the ks
    // waves of a tile group take steps b_*ks*U + kp*U + [0, U)); rows past
    // N, tile groups past the last and bytes past the row read zero.
    auto load_batch = [&](v4i(&buf)[U][R], int st_, int b_) {
        const int n0 = (st_ * slots + sg) * kTileRows * R;
        const int rows = max(0, min(kTileRows * R, N - n0));
        const auto rw = make_rsrc(packed + (size_t)min(n0, N) * rowbytes, (uint32_t)rows * rowbytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = b_ * ks * U + kp * U + u;
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
                                         [&] { load_batch(bcur, st, b); });
        }
#pragma unroll
        for (int m = 1; m < FM; ++m) {
            if (m < M) {
                LdsRowSink sink{q_lds + m * K, inv_sh + m, qsum_sh + m};
                block_act_quant_row<8, LONG>(x + (size_t)m * K, gamma, eps, K, red, sink, [] {});
            }
        }
        __syncthreads();
        if (A.tg_first == 0) {
            for (int i = tid; i < M * K / 16; i += 256)
                reinterpret_cast<uint4 *>(A.q_out)[i] = reinterpret_cast<const uint4 *>(q_lds)[i];
            if (tid < M) {
                A.inv_out[tid] = inv_sh[tid];
                A.qsum_out[tid] = qsum_sh[tid];
            }
        }
    } else if constexpr (MODE == 1) {
        const uint4 *src = reinterpret_cast<const uint4 *>(q + (size_t)m0 * K);
        for (int i = tid; i < mg * K / 16; i += 256)
            reinterpret_cast<uint4 *>(q_lds)[i] = src[i];
        load_batch(bcur, st, b);
        __syncthreads();
    } else {
        load_batch(bcur, st, b);
    }

    for (;;) {
        int st2 = st, b2 = b + 1;
        if (b2 == nb) {
            st2 += A.tg_stride;
            b2 = 0;
        }
        const bool more = st2 < nset;
        if (more) load_batch(bnxt, st2, b2);

        // Contract the current batch.
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = b * ks * U + kp * U + u;
            const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
            const bool kv = (s < nsteps) && (cb < rowbytes);
            // k of this lane's chunk: block cb / 32, half (cb / 16) % 2.
            const int kb = (int)(cb / 32) * kBlockWeights + 16 * (int)((cb / 16) & 1);
            v4i a[TH][4];
#pragma unroll
            for (int h = 0; h < TH; ++h) {
                const int t = 8 * h + r8;  // token (group-relative)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if constexpr (MODE == 2) {
                        const bool av = kv && t < mg;
                        a[h][g] = buf_load16(rq, av ? (uint32_t)(t * K + kb + 32 * g) : kOOB);
                    } else {
                        // In-bounds LDS rows without zero-fill: tokens past
                        // the group read its last row (their D rows are never
                        // stored), chunks past K read chunk 0 (their weight
                        // bytes are zeros).
                        const int tc = min(t, mg - 1);
                        a[h][g] = *reinterpret_cast<const v4i *>(q_lds + tc * K + (kv ? kb : 0) +
                                                                 32 * g);
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
            // Set done: sum the fields, then the ks waves of each tile group.
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
            const int tg = st * slots + sg;
            const int l = lane;
            if (kp == 0 && tg < ntg && (l & 8) == 0 && l < 24) {
#pragma unroll
                for (int h = 0; h < TH; ++h)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        v4i t = part[wid][h][r][l] + part[wid][h][r][l + 40];
                        for (int w = 1; w < ks; ++w)
                            t += part[wid + w][h][r][l] + part[wid + w][h][r][l + 40];
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
        st = st2;
        b = b2;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r) bcur[u][r] = bnxt[u][r];
    }
}

// Streaming form of the same contraction for MODE 0 and 1 (activations in
// LDS).  The weight batches are not loaded into registers but copied by
// LDS-direct buffer loads into a ring of D batch slots private to each
// wave: D - 1 batches are in flight while one is contracted, so a wave
// keeps D - 1 times as many weight bytes in flight as the register form
// without spending registers on them.  Lane l of a copy writes its 16 bytes
// at slot + 16 l, i.e. in exactly the lane order the contraction reads them
// back (one contiguous, conflict-free 1 KB read per 8 rows x 128 bytes), and
// since each wave reads only what it copied, a wait on its own vmcnt is all
// the ordering needed.  Every copy is an LDS-direct load without a register
// result, so the compiler can neither move nor drop one and the explicit
// waits count them exactly; batches past the end are range-checked to read
// nothing, so every batch waits on the same count.
template <int R, int U, int D, int MODE, bool OUT_Y, int FM, bool LONG, int TH>
__device__ __forceinline__ void gemv_ring_body(const GemvArgs &A) {
    static_assert(MODE == 0 || MODE == 1, "activations must be in LDS");
    static_assert(D >= 2 && D <= 8 && (D - 1) * U * R < 64, "ring depth");
    extern __shared__ __align__(16) int8_t q_lds[];
    // One LDS object per slot (rows: waves), so that the compiler's own
    // LDS-DMA tracking tells the slots apart.
    constexpr int SZ = U * R * 1024;
    __shared__ __align__(16) int8_t s0[kW][SZ], s1[kW][SZ], s2[D > 2 ? kW : 1][D > 2 ? SZ : 16],
        s3[D > 3 ? kW : 1][D > 3 ? SZ : 16], s4[D > 4 ? kW : 1][D > 4 ? SZ : 16],
        s5[D > 5 ? kW : 1][D > 5 ? SZ : 16], s6[D > 6 ? kW : 1][D > 6 ? SZ : 16],
        s7[D > 7 ? kW : 1][D > 7 ? SZ : 16];
    const float *__restrict__ x = A.x;
    const float *__restrict__ gamma = A.gamma;
    const int8_t *__restrict__ q = A.q;
    const float *__restrict__ inv = A.inv;
    const int32_t *__restrict__ qsum = A.qsum;
    const uint8_t *__restrict__ packed = A.packed;
    float *__restrict__ y = A.y;
    int32_t *__restrict__ acc_out = A.acc_out;
    const float eps = A.eps, w_scale = A.w_scale;
    const int M = A.M, K = A.K, N = A.N;
    __shared__ float red[kRedWords];
    __shared__ float inv_sh[16];
    __shared__ int qsum_sh[16];
    __shared__ v4i part[kW][TH][R][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps derived resources scalar
    const int r8 = lane & 7;    // weight row within the tile (load role)
    const int ch = lane >> 3;   // 16-byte chunk within the 128-byte step
    const int m0 = A.m0;
    const int mg = min(16, M - m0);

    const uint32_t rowbytes = (uint32_t)K / 4;
    const int nsteps = (int)((rowbytes + kStep - 1) / kStep);
    const int ks = A.ks;
    const int slots = kW / ks;
    const int sg = wid / ks, kp = wid % ks;
    const int nb = (nsteps + ks * U - 1) / (ks * U);
    const int ntg = (N + kTileRows * R - 1) / (kTileRows * R);
    const int nset = (ntg + slots - 1) / slots;

    // Copy batch (st_, b_) of this wave's tile group into ring slot `slot`.
    auto issue = [&](int8_t *slot, int st_, int b_) {
        const int n0 = (st_ * slots + sg) * kTileRows * R;
        const int rows = st_ < nset ? max(0, min(kTileRows * R, N - n0)) : 0;
        const auto rw = make_rsrc(packed + (size_t)min(n0, N) * rowbytes, (uint32_t)rows * rowbytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = b_ * ks * U + kp * U + u;
            const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
            const bool kv = (s < nsteps) && (cb < rowbytes);
#pragma unroll
            for (int r = 0; r < R; ++r)
                buf_load16_lds(rw, slot + (u * R + r) * 1024,
                               kv ? (uint32_t)(kTileRows * r + r8) * rowbytes + cb : kOOB, 0);
        }
    };
    // Issue-side cursor: the next batch to copy.
    int ist = A.tg_first, ib = 0;
    auto advance = [&](int &st_, int &b_) {
        if (++b_ == nb) {
            b_ = 0;
            st_ += A.tg_stride;
        }
    };
    auto slot_of = [&](auto I) -> int8_t * {
        constexpr int i = decltype(I)::value;
        if constexpr (i == 0) return s0[wid];
        else if constexpr (i == 1) return s1[wid];
        else if constexpr (i == 2) return s2[wid];
        else if constexpr (i == 3) return s3[wid];
        else if constexpr (i == 4) return s4[wid];
        else if constexpr (i == 5) return s5[wid];
        else if constexpr (i == 6) return s6[wid];
        else return s7[wid];
    };
    auto issue_next = [&](auto I) {
        issue(slot_of(I), ist, ib);
        advance(ist, ib);
    };
    auto prologue_issue = [&] {
        unroll_ic([&](auto I) {
            if constexpr (decltype(I)::value < D - 1) issue_next(I);
        }, std::make_integer_sequence<int, D>{});
    };

    if constexpr (MODE == 0) {
        // x and gamma loads go first, the first D - 1 weight batches right
        // behind them, so the normalisation never waits for the weights.
        {
            LdsRowSink sink{q_lds, inv_sh, qsum_sh};
            block_act_quant_row<8, LONG>(x, gamma, eps, K, red, sink, prologue_issue);
        }
#pragma unroll
        for (int m = 1; m < FM; ++m) {
            if (m < M) {
                LdsRowSink sink{q_lds + m * K, inv_sh + m, qsum_sh + m};
                block_act_quant_row<8, LONG>(x + (size_t)m * K, gamma, eps, K, red, sink, [] {});
            }
        }
        lds_barrier();
        if (A.tg_first == 0) {
            for (int i = tid; i < M * K / 16; i += 256)
                reinterpret_cast<uint4 *>(A.q_out)[i] = reinterpret_cast<const uint4 *>(q_lds)[i];
            if (tid < M) {
                A.inv_out[tid] = inv_sh[tid];
                A.qsum_out[tid] = qsum_sh[tid];
            }
        }
    } else {
        // The token group's q rows, inv and qsum go to LDS before any weight
        // copy is issued, so no later wait on them drains the ring.
        const uint4 *src = reinterpret_cast<const uint4 *>(q + (size_t)m0 * K);
        for (int i = tid; i < mg * K / 16; i += 256)
            reinterpret_cast<uint4 *>(q_lds)[i] = src[i];
        if (tid < mg) {
            if (OUT_Y) inv_sh[tid] = inv[m0 + tid];  // inv is absent for int32 output
            qsum_sh[tid] = qsum[m0 + tid];
        }
        __syncthreads();
        prologue_issue();
    }

    v4i acc[4][TH][R];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h = 0; h < TH; ++h)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[g][h][r] = v4i{0, 0, 0, 0};

    int st = A.tg_first;  // compute-side cursor
    int b = 0;
    bool live = st < nset;
    // Contract batch (st, b) from ring slot `slot`; on the last batch of a
    // set, reduce and write the set's outputs.
    auto contract = [&](const int8_t *slot) {
        v4i bw[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                bw[u][r] = *reinterpret_cast<const v4i *>(slot + (u * R + r) * 1024 + 16 * lane);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = b * ks * U + kp * U + u;
            const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
            const bool kv = (s < nsteps) && (cb < rowbytes);
            const int kb = (int)(cb / 32) * kBlockWeights + 16 * (int)((cb / 16) & 1);
            v4i a[TH][4];
#pragma unroll
            for (int h = 0; h < TH; ++h) {
                // (in-bounds rows, no zero-fill: as in the register form)
                const int tc = min(8 * h + r8, mg - 1);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    a[h][g] = *reinterpret_cast<const v4i *>(q_lds + tc * K + (kv ? kb : 0) +
                                                             32 * g);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const v4i bf = unpack_field(bw[u][r], g);
#pragma unroll
                    for (int h = 0; h < TH; ++h) acc[g][h][r] = mfma16(a[h][g], bf, acc[g][h][r]);
                }
        }
        if (b == nb - 1) {
#pragma unroll
            for (int h = 0; h < TH; ++h)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    part[wid][h][r][lane] =
                        (acc[0][h][r] + acc[1][h][r]) + (acc[2][h][r] + acc[3][h][r]);
#pragma unroll
                    for (int g = 0; g < 4; ++g) acc[g][h][r] = v4i{0, 0, 0, 0};
                }
            lds_barrier();
            const int tg = st * slots + sg;
            const int l = lane;
            if (kp == 0 && tg < ntg && (l & 8) == 0 && l < 24) {
#pragma unroll
                for (int h = 0; h < TH; ++h)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        v4i t = part[wid][h][r][l] + part[wid][h][r][l + 40];
                        for (int w = 1; w < ks; ++w)
                            t += part[wid + w][h][r][l] + part[wid + w][h][r][l + 40];
                        const int n = tg * kTileRows * R + kTileRows * r + (l & 7);
                        if (n < N) {
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const int mloc = 8 * h + 4 * (l >> 4) + c;
                                if (mloc < mg) {
                                    const int m = m0 + mloc;
                                    const int qs = qsum_sh[mloc];
                                    const int v = t[c] - qs;
                                    if (OUT_Y) {
                                        const float iv = inv_sh[mloc];
                                        y[(size_t)m * N + n] = (float)v * (w_scale / iv);
                                    } else {
                                        acc_out[(size_t)m * N + n] = v;
                                    }
                                }
                            }
                        }
                    }
            }
            lds_barrier();
        }
        advance(st, b);
        live = st < nset;
    };

    // Batch j sits in slot j % D.  At batch j: copy batch j + D - 1 into the
    // slot batch j - 1 was read from, wait for batch j's own copies (the
    // D - 1 later batches may stay in flight), contract it.
    constexpr int kPend = (D - 1) * U * R;
    while (live) {
        unroll_ic([&](auto I) {
            constexpr int i = decltype(I)::value;
            if (!live) return;
            issue_next(ic<(i + D - 1) % D>{});
            wait_vmcnt<kPend>();
            contract(slot_of(I));
        }, std::make_integer_sequence<int, D>{});
    }
    // Drain the trailing (empty) copies before the workgroup's LDS is
    // released.
    wait_vmcnt<0>();
}

// Separate-quantisation forms (MODE 1, 2): one problem, token groups on
// blockIdx.y.
template <int R, int U, int D, int MODE, bool OUT_Y, int TH>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs A) {
    A.m0 = blockIdx.y * 16;
    A.tg_first = blockIdx.x;
    A.tg_stride = gridDim.x;
    if constexpr (MODE == 2)
        gemv_body<R, U, 2, OUT_Y, 0, false, TH>(A);
    else
        gemv_ring_body<R, U, D, 1, OUT_Y, 0, false, TH>(A);
}

// Fused form (MODE 0) over a batch of independent decode BitLinears: the
// workgroups [wg_begin, wg_begin + wg_count) serve problem i.  One launch
// covers a whole decode step.
constexpr int kMaxBatch = 8;
struct FusedProblem {
    const float *x;
    const float *gamma;
    const uint8_t *packed;
    float *y;
    int8_t *q_out;
    float *inv_out;
    int32_t *qsum_out;
    float eps;
    float w_scale;
    int M, K, N;
    int wg_begin, wg_count;
    int ks;
};
struct FusedBatch {
    FusedProblem p[kMaxBatch];
    int count;
};

template <int R, int U, int D, int FM, bool LONG>
__global__ __launch_bounds__(256) void gemv_fused_kernel(FusedBatch B) {
    // The batch is the kernel's only argument: read it in place from the
    // kernel-argument segment (constant memory, wave-uniform addresses, so
    // scalar loads) instead of from a copy of the by-value parameter.
    const FusedBatch *Bk = reinterpret_cast<const FusedBatch *>(
        (const void *)__builtin_amdgcn_kernarg_segment_ptr());
    int i = 0;
    const int count = Bk->count;
    for (int t = 1; t < count; ++t)
        if ((int)blockIdx.x >= Bk->p[t].wg_begin) i = t;
    const FusedProblem &P = Bk->p[i];
    GemvArgs A;
    A.x = P.x;
    A.gamma = P.gamma;
    A.q = P.q_out;
    A.inv = P.inv_out;
    A.qsum = P.qsum_out;
    A.packed = P.packed;
    A.y = P.y;
    A.acc_out = nullptr;
    A.q_out = P.q_out;
    A.inv_out = P.inv_out;
    A.qsum_out = P.qsum_out;
    A.eps = P.eps;
    A.w_scale = P.w_scale;
    A.M = P.M;
    A.K = P.K;
    A.N = P.N;
    A.m0 = 0;
    A.tg_first = (int)blockIdx.x - P.wg_begin;
    A.tg_stride = P.wg_count;
    A.ks = P.ks;
    gemv_ring_body<R, U, D, 0, true, FM, LONG, 1>(A);
}

struct Shape {
    int R, U, D;  // tiles per group, 128-byte steps per batch, ring depth
};
// Launch-shape table; every entry computes bit-identical results.  A wave's
// ring holds D * U * R KB (at most 24 KB, so a workgroup's ring plus the
// largest staged activation block fits the LDS).
constexpr Shape kShapes[] = {{1, 2, 4}, {1, 2, 8}, {1, 4, 4}, {2, 2, 4},
                             {1, 1, 8}, {2, 4, 3}, {1, 4, 6}, {4, 2, 3}};
constexpr bool rings_fit() {
    for (const Shape &h : kShapes)
        if (h.R * h.U * h.D > 24 || h.D < 2) return false;
    return true;
}
static_assert(rings_fit(), "ring size");
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

// LDS a workgroup may use on this device (queried once; every device this
// library runs on is a gfx950).
size_t max_lds_per_block() {
    static const size_t n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            return (size_t)64 * 1024;
        return (size_t)v;
    }();
    return n;
}

// Static LDS of a kernel (a property of its code object, queried once).
template <auto Kernel>
size_t static_lds() {
    static const size_t n = [] {
        hipFuncAttributes a{};
        if (hipFuncGetAttributes(&a, reinterpret_cast<const void *>(Kernel)) != hipSuccess)
            return (size_t)-1;
        return a.sharedSizeBytes;
    }();
    return n;
}

// Whether Kernel with `dyn` bytes of dynamic LDS fits one workgroup.
template <auto Kernel>
bool lds_fits(size_t dyn) {
    const size_t st = static_lds<Kernel>();
    return st != (size_t)-1 && st + dyn <= max_lds_per_block();
}

// Smallest K split (waves per tile group) that still gives each of `wgs`
// workgroups a set of tile groups: fewer waves per tile group means longer
// per-wave streams and more tile groups in flight.
int pick_ks(int64_t ntg, int64_t wgs) {
    for (int ks = 1; ks < kW; ks *= 2)
        if ((ntg + kW / ks - 1) / (kW / ks) >= wgs) return ks;
    return kW;
}

template <int R, int U, int D, int MODE, bool OUT_Y, int TH>
hipError_t launch_sep(const int8_t *q, const float *inv, const int32_t *qsum,
                      const uint8_t *packed, float w_scale, int64_t M, int64_t K, int64_t N,
                      float *y, int32_t *acc, hipStream_t s) {
    const int64_t ntg = (N + kTileRows * R - 1) / (kTileRows * R);
    const unsigned gy = (unsigned)((M + 15) / 16);
    const int64_t mg = M < 16 ? M : 16;
    const size_t lds = MODE == 1 ? (size_t)(mg * K) : 0;
    // One wave of co-resident workgroups walks all tile groups.
    auto kern = gemv_kernel<R, U, D, MODE, OUT_Y, TH>;
    if (!lds_fits<gemv_kernel<R, U, D, MODE, OUT_Y, TH>>(lds)) return hipErrorInvalidConfiguration;
    const int64_t cap = std::max<int64_t>(1, (int64_t)cu_count() * resident_per_cu(kern, lds) / gy);
    const int ks = pick_ks(ntg, cap);
    const int64_t nset = (ntg + kW / ks - 1) / (kW / ks);
    // Every workgroup walks the same number of sets: a grid of cap with a
    // few workgroups taking one set more leaves the device underused for
    // that last set.
    const int64_t per = (nset + cap - 1) / cap;
    const unsigned gx = (unsigned)((nset + per - 1) / per);
    GemvArgs A{};
    A.ks = ks;
    A.q = q;
    A.inv = inv;
    A.qsum = qsum;
    A.packed = packed;
    A.y = y;
    A.acc_out = acc;
    A.w_scale = w_scale;
    A.M = (int)M;
    A.K = (int)K;
    A.N = (int)N;
    hipLaunchKernelGGL(kern, dim3(gx, gy), dim3(256), lds, s, A);
    return hipGetLastError();
}

template <int R, int U, int D>
hipError_t launch_shape_sep(const int8_t *q, const float *inv, const int32_t *qsum,
                            const uint8_t *packed, float w_scale, int64_t M, int64_t K, int64_t N,
                            float *y, int32_t *acc, int mode, hipStream_t s) {
#define BL_ONE(D_, MODE, TH)                                                                     \
    return y ? launch_sep<R, U, D_, MODE, true, TH>(q, inv, qsum, packed, w_scale, M, K, N, y,   \
                                                    acc, s)                                      \
             : launch_sep<R, U, D_, MODE, false, TH>(q, inv, qsum, packed, w_scale, M, K, N, y,  \
                                                     acc, s);
    const bool two = M > 8;
    if (mode == 1) {
        // The staged form keeps the token group's q rows next to the weight
        // ring in LDS; where the two do not fit one workgroup, q is read
        // from global memory instead.
        const size_t dyn = (size_t)((M < 16 ? M : 16) * K);
        const bool fits = two ? (y ? lds_fits<gemv_kernel<R, U, D, 1, true, 2>>(dyn)
                                   : lds_fits<gemv_kernel<R, U, D, 1, false, 2>>(dyn))
                              : (y ? lds_fits<gemv_kernel<R, U, D, 1, true, 1>>(dyn)
                                   : lds_fits<gemv_kernel<R, U, D, 1, false, 1>>(dyn));
        if (fits) {
            if (two) { BL_ONE(D, 1, 2) }
            BL_ONE(D, 1, 1)
        }
    }
    if (two) { BL_ONE(0, 2, 2) }
    BL_ONE(0, 2, 1)
#undef BL_ONE
}

// Fused launch over `count` problems (count <= kMaxBatch): workgroups are
// shared out in proportion to each problem's weight bytes, within the
// number that fit on the device at once.
template <int R, int U, int D, int FM, bool LONG>
hipError_t launch_fused(const FusedDecode *d, int count, hipStream_t s) {
    int64_t max_mk = 1;
    for (int i = 0; i < count; ++i) max_mk = std::max<int64_t>(max_mk, d[i].M * d[i].K);
    const size_t lds = (size_t)max_mk;
    auto kern = gemv_fused_kernel<R, U, D, FM, LONG>;
    if (!lds_fits<gemv_fused_kernel<R, U, D, FM, LONG>>(lds)) return hipErrorInvalidConfiguration;
    const int64_t cap = std::max<int64_t>(count, (int64_t)cu_count() * resident_per_cu(kern, lds));
    int64_t ntg[kMaxBatch], total_tg = 0;
    double bytes[kMaxBatch], total_bytes = 0.0;
    for (int i = 0; i < count; ++i) {
        ntg[i] = (d[i].N + kTileRows * R - 1) / (kTileRows * R);
        total_tg += ntg[i];
        bytes[i] = (double)d[i].N * (double)d[i].K;
        total_bytes += bytes[i];
    }
    FusedBatch B{};
    B.count = count;
    int64_t begin = 0;
    for (int i = 0; i < count; ++i) {
        int64_t w = total_tg <= cap ? ntg[i]
                                    : (int64_t)((double)cap * bytes[i] / total_bytes);
        w = std::max<int64_t>(1, std::min(w, ntg[i]));
        const int ks = pick_ks(ntg[i], w);
        const int64_t nset = (ntg[i] + kW / ks - 1) / (kW / ks);
        w = std::min(w, nset);
        FusedProblem &P = B.p[i];
        P.ks = ks;
        P.x = d[i].x;
        P.gamma = d[i].gamma;
        P.packed = d[i].packed;
        P.y = d[i].y;
        P.q_out = d[i].q;
        P.inv_out = d[i].inv;
        P.qsum_out = d[i].qsum;
        P.eps = d[i].eps;
        P.w_scale = d[i].w_scale;
        P.M = (int)d[i].M;
        P.K = (int)d[i].K;
        P.N = (int)d[i].N;
        P.wg_begin = (int)begin;
        P.wg_count = (int)w;
        begin += w;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)begin), dim3(256), lds, s, B);
    return hipGetLastError();
}

template <int R, int U, int D>
hipError_t launch_shape_fused(const FusedDecode *d, int count, hipStream_t s) {
    bool lng = false;
    int64_t max_m = 1;
    for (int i = 0; i < count; ++i) {
        lng = lng || d[i].K > 8 * 1024;
        max_m = std::max<int64_t>(max_m, d[i].M);
    }
    if (max_m == 1)
        return lng ? launch_fused<R, U, D, 1, true>(d, count, s)
                   : launch_fused<R, U, D, 1, false>(d, count, s);
    return lng ? launch_fused<R, U, D, kFuseMaxM, true>(d, count, s)
               : launch_fused<R, U, D, kFuseMaxM, false>(d, count, s);
}

}  // namespace

// Variants 1..kNumShapes: the persistent streaming form with that launch
// shape; kNumShapes + 1: the one-shot form (gemv_shot.hip) where it applies,
// launch shape picked from the problems; kNumShapes + 1 + j: the one-shot
// form with its launch shape j (taken when every problem fits it).
constexpr int kShotVariants = kShotShapeCount + 1;
// Last variant: the rolling form of the one-shot kernel (where it applies).
constexpr int kRollVariant = kNumShapes + kShotVariants + 1;
int gemv_num_variants() { return kRollVariant; }

static int shot_shape_of(int variant) { return variant - kNumShapes - 1; }
static bool is_shot(int variant) {
    return variant > kNumShapes && variant <= kNumShapes + kShotVariants;
}

// Automatic choice of the persistent form's launch shape (measured best on
// the decode shapes of 2560- to 28672-wide layers).
// Persistent-form shape for M tokens: one tile per wave for one token, two
// up to 4 tokens, four beyond (each tile's activation fragments serve more
// rows as M grows; measured at K = 16384..28672).
static int auto_variant(int64_t M) { return M <= 1 ? 1 : M <= 4 ? 6 : 8; }

#define BL_GEMV_SWITCH(CALL)                                                  \
    switch (v) {                                                              \
        case 1: return CALL(kShapes[0].R, kShapes[0].U, kShapes[0].D);                      \
        case 2: return CALL(kShapes[1].R, kShapes[1].U, kShapes[1].D);                      \
        case 3: return CALL(kShapes[2].R, kShapes[2].U, kShapes[2].D);                      \
        case 4: return CALL(kShapes[3].R, kShapes[3].U, kShapes[3].D);                      \
        case 5: return CALL(kShapes[4].R, kShapes[4].U, kShapes[4].D);                      \
        case 6: return CALL(kShapes[5].R, kShapes[5].U, kShapes[5].D);                      \
        case 7: return CALL(kShapes[6].R, kShapes[6].U, kShapes[6].D);                      \
        case 8: return CALL(kShapes[7].R, kShapes[7].U, kShapes[7].D);                      \
        default: return hipErrorInvalidValue;                                 \
    }

hipError_t launch_gemv(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M, int64_t K, int64_t N,
                       float *y, int32_t *acc, int variant, hipStream_t s) {
    const int64_t mg = M < 16 ? M : 16;
    const int mode = mg * K <= kGemvStageMaxLds ? 1 : 2;
    const ShotDecode d{q, inv, qsum, packed, y, acc, w_scale, M, K, N};
    if (variant == kRollVariant && roll_supported(M, K)) return launch_gemv_roll(&d, 1, s);
    if (variant == kRollVariant) variant = 0;
    // Automatic: the one-shot form where all of its workgroups are resident
    // at once, else the rolling form (measured faster than the one-shot form
    // over several rounds and than the persistent form: M = 1..8 at the 70B
    // FFN shapes, 1.1-1.5x), else the one-shot form for rows up to 16384
    // and the persistent form beyond.
    if (variant == 0) {
        const bool shot = M * K <= kShotSingleMaxQ && K <= 16384 && shot_supported(M, K);
        if (shot && shot_rounds(&M, &K, &N, 1, false) == 1) variant = kNumShapes + 1;
        else if (roll_supported(M, K)) return launch_gemv_roll(&d, 1, s);
        else if (shot) variant = kNumShapes + 1;
    }
    if (is_shot(variant) && shot_supported(M, K))
        return launch_gemv_shot(&d, 1, shot_shape_of(variant), s);
    const int v = variant > 0 && variant <= kNumShapes ? variant : auto_variant(M);
#define BL_SEP(R_, U_, D_) \
    launch_shape_sep<R_, U_, D_>(q, inv, qsum, packed, w_scale, M, K, N, y, acc, mode, s)
    BL_GEMV_SWITCH(BL_SEP)
#undef BL_SEP
}

hipError_t launch_gemv_fused(const FusedDecode *d, int count, int variant, hipStream_t s) {
    bool fits = true;
    int64_t M[8], K[8], N[8];
    const bool glu = count > 0 && d[0].u != nullptr;
    if (variant == kRollVariant) {
        bool roll = count <= 8;
        for (int i = 0; i < count; ++i)
            roll = roll && roll_fused_supported(d[i].M, d[i].K) && !d[i].u && d[i].io == kIoF32;
        if (roll) return launch_gemv_roll_fused(d, count, s);
        variant = 0;
    }
    for (int i = 0; i < count; ++i) {
        fits = fits && shot_fused_supported(d[i].M, d[i].K);
        if (i < 8) {
            M[i] = d[i].M;
            K[i] = d[i].K;
            N[i] = d[i].N;
        }
    }
    // A few tokens (some problem with 2..kFewFusedMaxM rows): the one-shot
    // form whose quads quantise rows side by side, when it holds the set in
    // one round; else the one-token problems go out fused on their own and
    // the others as the batched quantisation + one-shot / rolling pair.
    int64_t mmax = 0;
    for (int i = 0; i < count && i < 8; ++i) mmax = std::max<int64_t>(mmax, d[i].M);
    if (variant == 0 && mmax >= 2 && count <= 8 && !glu) {
        bool all_f32 = true;
        for (int i = 0; i < count; ++i) all_f32 = all_f32 && d[i].io == kIoF32;
        if (all_f32 && few_fused_one_round(M, K, N, count))
            return launch_gemv_shot_fused(d, count, kFewFusedShapeVariant, s);
        bool pairable = all_f32 && mmax <= kFewFusedMaxM;
        for (int i = 0; i < count; ++i)
            pairable = pairable && (d[i].M == 1 || (d[i].K <= kActQuantBatchMaxK &&
                                                    shot_supported(d[i].M, d[i].K)));
        if (pairable) {
            FusedDecode one[8];
            ActQuantDesc aq[8];
            ShotDecode sd[8];
            int n1 = 0, n2 = 0;
            for (int i = 0; i < count; ++i) {
                const FusedDecode &f = d[i];
                if (f.M == 1) {
                    one[n1++] = f;
                } else {
                    aq[n2] = ActQuantDesc{f.x, f.gamma, f.eps, f.M, f.K, f.q, f.inv, f.qsum};
                    sd[n2] = ShotDecode{f.q, f.inv, f.qsum, f.packed, f.y, nullptr, f.w_scale,
                                        f.M, f.K, f.N};
                    ++n2;
                }
            }
            if (n1 > 0)
                if (hipError_t e = launch_gemv_fused(one, n1, 0, s)) return e;
            if (hipError_t e = launch_act_quant_batch(aq, n2, s)) return e;
            return launch_gemv_shot_auto(sd, n2, s);
        }
    }
    // Automatic: the one-shot form when all of its workgroups fit on the
    // device at once and every row is held in registers by the block form
    // (K <= 8192); else, one token per problem, the rolling form (its
    // 1024-thread quantisation holds rows up to 32768: faster than the
    // one-shot form for longer rows and than the persistent form, measured
    // on the 70B FFN shapes); else the one-shot form when it fits, else the
    // persistent form.
    bool roll = variant == 0 && count <= 8 && !glu;
    int64_t kmax = 0;
    for (int i = 0; i < count && i < 8; ++i) {
        roll = roll && roll_fused_supported(d[i].M, d[i].K) && d[i].io == kIoF32;
        kmax = std::max<int64_t>(kmax, d[i].K);
    }
    const bool fits_one = fits && count <= 8 && shot_rounds(M, K, N, count, true, glu) == 1;
    if (variant == 0 && roll && !(fits_one && kmax <= 8192)) return launch_gemv_roll_fused(d, count, s);
    const bool shot = fits && count <= 8 && (is_shot(variant) || (variant == 0 && fits_one));
    if (shot)
        return launch_gemv_shot_fused(d, count, is_shot(variant) ? shot_shape_of(variant) : 0, s);
    // The persistent form reads and writes fp32 activations only.
    for (int i = 0; i < count; ++i)
        if (d[i].io != kIoF32 || d[i].u) return hipErrorInvalidValue;
    // (fused: one tile per wave, the shape measured for one token)
    const int v = variant > 0 && variant <= kNumShapes ? variant : 1;
#define BL_FUSED(R_, U_, D_) launch_shape_fused<R_, U_, D_>(d, count, s)
    BL_GEMV_SWITCH(BL_FUSED)
#undef BL_FUSED
}

#undef BL_GEMV_SWITCH

hipError_t launch_gemv_shot_auto(const ShotDecode *d, int count, hipStream_t s) {
    int64_t M[8], K[8], N[8];
    bool roll = count >= 1 && count <= 8;
    for (int i = 0; i < count && i < 8; ++i) {
        M[i] = d[i].M;
        K[i] = d[i].K;
        N[i] = d[i].N;
        roll = roll && roll_supported(d[i].M, d[i].K) && d[i].io == kIoF32;
    }
    if (roll && shot_rounds(M, K, N, count, false) != 1) return launch_gemv_roll(d, count, s);
    return launch_gemv_shot(d, count, 0, s);
}

}  // namespace bl
