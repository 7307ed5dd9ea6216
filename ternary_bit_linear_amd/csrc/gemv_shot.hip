// gemv_shot.hip -- one-shot decode contraction (gfx950).
//
// acc[m][n] = sum_k code(n, k) * q[m][k] - qsum[m], then optionally
// y[m][n] = (float)acc * (w_scale / inv[m]), for M <= 8 tokens whose int8
// activations are in global memory, or (fused form, M <= 4) whose q, inv
// and qsum each workgroup computes from x, gamma and eps (RMSNorm + absmax
// int8 quantisation).
// [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU FFN":
// the vec_dot over I2_S codes and int8 activations, codes offset by the
// activation sum; every output must be written.  HF-38087: RMSNorm on the
// activations before their quantisation.]
//
// Design.  Each workgroup owns one set of weight rows (W / ks waves' worth,
// a wave holding R tiles of 8 consecutive rows, ks waves splitting each
// tile group's K range) for the whole of K, and runs once: it issues every
// load it will need at the start -- the activation block (or x and gamma)
// and all of its weight batches, the weights as LDS-direct buffer loads
// (lane i of a load writes bytes [16 i, 16 i + 16) after the wave's base
// address, so no registers are held) -- then contracts batch after batch as
// each lands, reduces the ks partial tiles through LDS, writes its outputs
// and exits.  With no loop around the loads, a workgroup keeps its whole
// share in flight from its first instruction.  The host picks the launch
// shape (batches per wave, tiles per wave, waves per workgroup) so that
// every workgroup of the launch is resident at once where it can be: a
// problem set that fits in one round streams near the rate of a plain read
// of the same bytes, where a persistent loop with a deep ring stays ~15%
// below it.  Larger fused sets take the persistent form (gemv.hip).
//
// The arithmetic is the decode route's: the 16 bytes a lane copies hold,
// per 2-bit field g, the codes of 16 consecutive k of one weight row (row
// l % 8, chunk l / 8 of a 128-byte step); shifted and masked they are the
// B operand of v_mfma_i32_16x16x64_i8 whose 16 columns are 8 rows x 2 chunk
// parities, and the A operand holds the tokens in both halves of its 16 rows
// with the matching chunk; one lane + 40 add joins the two parities.
#include <atomic>
#include <climits>

#include "common.hpp"

namespace bl {
namespace {

constexpr int kMaxKs = 4;      // waves splitting one tile group's K range, at most
constexpr int kTileRows = 8;   // weight rows per tile
constexpr int kStep = 128;     // packed bytes of a row per step (512 k)
constexpr int kU = 2;          // steps per batch
constexpr int kMaxShotM = 8;

struct ShotProblem {
    const int8_t *q;       // activations (FM == 0)
    const float *inv;
    const int32_t *qsum;
    const float *x;        // fused normalisation (FM > 0)
    const float *gamma;
    int8_t *q_out;         // fused: q / inv / qsum, written by the first workgroup
    float *inv_out;
    int32_t *qsum_out;
    const uint8_t *packed;
    float *y;
    int32_t *acc;
    float eps;
    float w_scale;
    int M, K, N;
    int wg_begin;          // first workgroup of this problem
    int ks_log;            // log2 of the K split: 0..2 (one-shot), 0..4 (rolling)
    const float *u;        // GLU: up rows (the input row is relu2_mul(x, u))
};
constexpr int kMaxShotBatch = 8;
struct ShotBatch {
    ShotProblem p[kMaxShotBatch];
};
static_assert(alignof(ShotBatch) == 8, "the batch follows eight ints in the argument segment");

// q and inv of one token row into LDS and, for the problem's first
// workgroup (gq non-null), also into global memory -- straight from
// registers, so that no LDS read of them has to wait for the weight loads
// in flight.  The activation sum is left as four per-wave partials in LDS
// (qpart): the epilogue adds them after the barrier that publishes q, so its
// block reduction is not on the path to the first MFMA.
struct ShotRowSink {
    static constexpr bool kDeferSum = true;
    int8_t *q;
    float *inv;
    int *qpart;  // [4]
    int8_t *gq;
    float *ginv;
    __device__ void store_q(int k, uint32_t v) {
        *reinterpret_cast<uint32_t *>(q + k) = v;
        if (gq) *reinterpret_cast<uint32_t *>(gq + k) = v;
    }
    __device__ void store_inv(float iv) {
        *inv = iv;
        if (gq) *ginv = iv;
    }
    __device__ void store_qsum_part(int w, int qs) { qpart[w] = qs; }
};

// Sum over the four fields of per-field accumulators of scaled codes
// (unpack_scaled): each is an exact multiple of its scale.
__device__ __forceinline__ v4i field_sum(const v4i (&a)[4]) {
    return (a[0] + (a[1] >> kFieldShift[1])) + ((a[2] >> kFieldShift[2]) + a[3]);
}

// NB: weight batches (of kU 128-byte steps) per wave; the host picks ks so
// that a wave's share of a row fits NB batches.  R: tiles of 8 rows per wave
// (a wave's rows are 8 R consecutive rows; every batch holds all R tiles'
// steps, so the activation fragments of a step serve R tiles).  FM: 0 takes q / inv / qsum
// from global memory; FM > 0 computes them in every workgroup from x, gamma
// and eps (M <= FM rows of K <= 1024 * CH, or streamed when LONG).
// b0..b7: first workgroup of each problem (INT_MAX past the last); they
// lead the argument list so that the build's kernel-argument preload puts
// them in scalar registers at wave launch, and the lookup costs no memory
// round trip.
// IO: storage type of x and y with the fused quantisation (float, bf16_t,
// _Float16): x is widened to fp32 as it is loaded, y rounded as it is
// stored.
// W: waves per workgroup, 4, 8 or 16.  The quantisation is the 256-thread
// block form; in a larger workgroup waves 4..W-1 issue their weights and
// meet its barriers, so a CU that holds one such workgroup normalises x once
// where several 4-wave workgroups would each do it.  In such a workgroup
// waves 0..3 issue their weights after the quantisation, past the barrier
// that publishes q: a wave that issues many loads stalls at the issue until
// the memory pipeline takes them, and the quantisation's barriers would make
// every wave wait for it.
template <int NB, int R, bool OUT_Y, int FM, int CH, bool LONG, bool GLU = false,
          typename IO = float, int W = 4>
__global__ __launch_bounds__(64 * W) void gemv_shot_kernel(int b0, int b1, int b2, int b3, int b4,
                                                        int b5, int b6, int b7, ShotBatch B) {
    static_assert(NB >= 1 && NB <= 8, "batches per wave");
    static_assert(R == 1 || R == 2 || R == 4, "tiles per wave");
    static_assert(kMaxShotBatch == 8, "one leading argument per problem");
    static_assert(W == 4 || W == 8 || W == 16, "waves per workgroup");
    static_assert(kU == 2, "shift forms below assume kU == 2");
    constexpr int LW = W == 16 ? 4 : W == 8 ? 3 : 2;  // log2(W)
    static_assert(FM >= 0 && FM <= kMaxShotM, "fused token rows");
    extern __shared__ __align__(16) int8_t q_lds[];
    // One LDS object per batch (rows: waves), so that the compiler's own
    // LDS-DMA tracking tells the batches apart and waits for each alone.
    constexpr int SZ = R * kU * 1024;  // one batch of one wave
    __shared__ __align__(16) int8_t w0[W][SZ], w1[NB > 1 ? W : 1][NB > 1 ? SZ : 16],
        w2[NB > 2 ? W : 1][NB > 2 ? SZ : 16], w3[NB > 3 ? W : 1][NB > 3 ? SZ : 16],
        w4[NB > 4 ? W : 1][NB > 4 ? SZ : 16], w5[NB > 5 ? W : 1][NB > 5 ? SZ : 16],
        w6[NB > 6 ? W : 1][NB > 6 ? SZ : 16], w7[NB > 7 ? W : 1][NB > 7 ? SZ : 16];
    __shared__ float red[kRedWords * (W > 4 ? W / 4 : 1)];  // one block per quad
    __shared__ float inv_sh[FM > 0 ? FM : 1];
    __shared__ int qpart_sh[FM > 0 ? FM : 1][4];  // per-wave partial sums of q

    // The batch is read in place from the kernel-argument segment (constant
    // memory, wave-uniform addresses, so scalar loads): every field of this
    // workgroup's problem in one round trip, all at once, before any other
    // work (a field read where it is first used would cost a round trip of
    // its own).
    (void)b0;
    const int bx = (int)blockIdx.x;
    const int pi = (bx >= b1) + (bx >= b2) + (bx >= b3) + (bx >= b4) + (bx >= b5) + (bx >= b6) +
                   (bx >= b7);
    const ShotBatch *Bk = reinterpret_cast<const ShotBatch *>(
        (const char *)__builtin_amdgcn_kernarg_segment_ptr() + 8 * sizeof(int));
    const ShotProblem P = Bk->p[pi];
    asm volatile("" ::"s"(P.q), "s"(P.inv), "s"(P.qsum), "s"(P.x), "s"(P.gamma), "s"(P.q_out),
                 "s"(P.inv_out), "s"(P.qsum_out), "s"(P.packed), "s"(P.y), "s"(P.acc), "s"(P.eps),
                 "s"(P.w_scale), "s"(P.M), "s"(P.K), "s"(P.N), "s"(P.wg_begin), "s"(P.ks_log));
    if constexpr (GLU) asm volatile("" ::"s"(P.u));
    const int M = P.M, K = P.K, N = P.N;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps derived resources scalar
    const int r8 = lane & 7;    // weight row within the tile (load role)
    const int ch = lane >> 3;   // 16-byte chunk within the 128-byte step
    const uint32_t rowbytes = (uint32_t)K / 4;
    const int nsteps = (int)((rowbytes + kStep - 1) / kStep);
    const int kl = P.ks_log;
    const int ks = 1 << kl;
    const int sg = wid >> kl, kp = wid & (ks - 1);
    const int nb = (nsteps + ks * kU - 1) >> (kl + 1);   // <= NB (kU == 2)
    const int st = bx - P.wg_begin;                     // this workgroup's set
    const int tg = (st << (LW - kl)) + sg;              // this wave's tile group
    const int n0 = tg * kTileRows * R;
    auto batch = [&](auto I) -> int8_t * {
        constexpr int b = decltype(I)::value;
        if constexpr (b == 0) return w0[wid];
        else if constexpr (b == 1) return w1[wid];
        else if constexpr (b == 2) return w2[wid];
        else if constexpr (b == 3) return w3[wid];
        else if constexpr (b == 4) return w4[wid];
        else if constexpr (b == 5) return w5[wid];
        else if constexpr (b == 6) return w6[wid];
        else return w7[wid];
    };

    // Every weight batch of this wave (past the end: range-checked to read
    // nothing, so the count of loads is the same for every wave).
    auto issue_weights = [&] {
        const int rows = max(0, min(kTileRows * R, N - n0));
        const auto rw = make_rsrc(P.packed + (size_t)min(n0, N) * rowbytes, (uint32_t)rows * rowbytes);
        unroll_ic([&](auto I) {
            constexpr int b = decltype(I)::value;
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int s = b * ks * kU + kp * kU + u;
                    const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
                    const bool kv = b < nb && s < nsteps && cb < rowbytes;
                    const uint32_t off = (uint32_t)(r * kTileRows + r8) * rowbytes + cb;
                    buf_load16_lds(rw, batch(I) + (r * kU + u) * 1024, kv ? off : kOOB, 0);
                }
            }
        }, std::make_integer_sequence<int, NB>{});
    };

    // Epilogue operands of this lane's tokens (m = 4 (lane / 16) + c), read
    // before any weight load so that no wait at the end drains behind them.
    int qs_pre[4];
    float iv_pre[4];
    if constexpr (FM == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = min(4 * (lane >> 4) + c, M - 1);
            qs_pre[c] = P.qsum[m];
            iv_pre[c] = OUT_Y ? P.inv[m] : 1.0f;
        }
    }

    if constexpr (FM == 0) {
        // 1. The activation block (M rows of K int8, contiguous), 1 KB per
        //    wave load, loads spread over the waves; 2. the weights.
        //    The barrier between them puts every activation load of the
        //    workgroup ahead of its weight loads in the compute unit's
        //    memory pipeline (requests leave it in order): issued
        //    interleaved, the activations would arrive only after the
        //    weights queued before them.
        const uint32_t qbytes = (uint32_t)(M * K);
        const auto rq = make_rsrc(P.q, qbytes);
        for (uint32_t c = (uint32_t)wid * 1024u; c < qbytes; c += W * 1024u)
            buf_load16_lds(rq, q_lds + c, c + 16u * lane, 0);
        __builtin_amdgcn_s_barrier();
        issue_weights();
        // 3. Own activation loads done (only weight loads may still be in
        //    flight), then every wave's: the block is complete in LDS.
        wait_vmcnt<NB * R * kU>();
        lds_barrier();
    } else {
        // 1. x and gamma of the first row go out first, the weights right
        //    behind them: a barrier after the x / gamma loads (rows held in
        //    registers) puts them ahead of every weight load of the
        //    workgroup in the memory pipeline, so they return at their own
        //    latency instead of after the weights queued before them;
        // 2. RMSNorm + quantisation of every row into LDS while the weights
        //    stream in.
        constexpr bool kLate = W > 4;  // quantising waves: weights after the quantisation
        constexpr bool kSync = !LONG;
        // In a larger workgroup (rows held in registers) each group of four
        // waves (a quad) quantises its own rows -- quad j rows j, j + W / 4,
        // ... -- its waves meeting on an LDS counter of their own instead of
        // workgroup barriers: the other waves, which may stall at the issue
        // of their weights, never hold a quantisation up, and the rows of a
        // few-token block are normalised side by side.  Otherwise waves 0..3
        // quantise every row in turn.
        constexpr bool kSpin = kSync && W > 4;
        constexpr int Q = kSpin ? W / 4 : 1;  // quads quantising rows
        const int quad = kSpin ? (wid >> 2) : 0;
        const int rows = min(M, FM);
        const bool quantises = kSpin ? quad < rows : (W == 4 || wid < 4);
        __shared__ int spin_sh[Q];
        if constexpr (kSpin) {
            // Zero, and visible to every wave past the first barrier below.
            if (tid < Q) spin_sh[tid] = 0;
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        }
        QuadSpin meet{&spin_sh[quad], 0};
        QuadSpin *const spin = kSpin ? &meet : nullptr;
        float *const qred = red + quad * kRedWords;
        if (quantises) {
            {
                const int m = quad;
                ShotRowSink sink{q_lds + m * K, inv_sh + m, qpart_sh[m],
                                 st == 0 ? P.q_out + (size_t)m * K : nullptr, P.inv_out + m};
                auto hook = [&] {
                    if constexpr (!kLate) issue_weights();
                };
                block_act_quant_row<CH, LONG, kSync, GLU, IO>(
                    reinterpret_cast<const IO *>(P.x) + (size_t)m * K, P.gamma, P.eps, K, qred,
                    sink, hook, GLU ? P.u + (size_t)m * K : nullptr, spin);
            }
#pragma unroll
            for (int i = 1; i < (FM + Q - 1) / Q; ++i) {
                const int m = quad + Q * i;
                if (m < rows) {
                    ShotRowSink sink{q_lds + m * K, inv_sh + m, qpart_sh[m],
                                     st == 0 ? P.q_out + (size_t)m * K : nullptr, P.inv_out + m};
                    block_act_quant_row<CH, LONG, false, GLU, IO>(
                        reinterpret_cast<const IO *>(P.x) + (size_t)m * K, P.gamma, P.eps, K,
                        qred, sink, [] {}, GLU ? P.u + (size_t)m * K : nullptr, spin);
                }
            }
        } else {
            // The other waves: the barrier behind the first rows' x / gamma
            // loads and their weights; with streamed rows also the barriers
            // of each row's block form.
            if constexpr (kSync) __builtin_amdgcn_s_barrier();
            issue_weights();
            if constexpr (!kSpin) {
#pragma unroll
                for (int m = 0; m < FM; ++m)
                    if (m < M) block_act_quant_row_barriers(P.gamma != nullptr, true);
            }
        }
        // (Published by a barrier: a count of the quantising waves polled
        // by the others measured slower.)
        lds_barrier();
        // The quantising waves of a larger workgroup issue their weights
        // only now, past the barrier that publishes q: an issue that stalls
        // then delays only their own contraction.
        if constexpr (kLate)
            if (quantises) issue_weights();
        // The problem's first workgroup also stores the rows' activation
        // sums (the partials are visible after the barrier).
        if (st == 0 && tid < M && tid < FM)
            P.qsum_out[tid] = (qpart_sh[tid][0] + qpart_sh[tid][1]) +
                              (qpart_sh[tid][2] + qpart_sh[tid][3]);
    }

    // 4. Contract each batch as it lands.  The activation fragments of the
    //    next batch are read from LDS while the current one is contracted.
    // A lane whose token row r8 is past M reads row M - 1 instead: those A
    // rows only reach D rows of tokens >= M, which are never stored.  A
    // chunk past K reads the row's first chunk: its weight bytes were loaded
    // as zeros (codes 0), so it adds nothing.  Every read is in bounds and
    // no fragment is cleared first.
    const int qrow = min(r8, M - 1) * K;
    auto read_q = [&](v4i(&a)[kU][4], int b) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int s = b * ks * kU + kp * kU + u;
            const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
            const bool kv = s < nsteps && cb < rowbytes;
            // k of this lane's chunk: block cb / 32, half (cb / 16) % 2.
            const int kb = kv ? (int)(cb / 32) * kBlockWeights + 16 * (int)((cb / 16) & 1) : 0;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                a[u][g] = *reinterpret_cast<const v4i *>(q_lds + qrow + kb + 32 * g);
        }
    };
    // The accumulators start at the first MFMAs (batch 0, step 0, which
    // every wave runs) with a zero addend, so no register is cleared on the
    // way from the quantisation to the first MFMA.
    v4i acc[R][4];
    v4i aq[2][kU][4];
    read_q(aq[0], 0);
    unroll_ic([&](auto I) {
        constexpr int b = decltype(I)::value;
        if (b >= nb) return;
        if (b + 1 < NB) read_q(aq[(b + 1) & 1], b + 1);
        wait_vmcnt<(NB - 1 - b) * R * kU>();
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const v4i bw =
                    *reinterpret_cast<const v4i *>(batch(I) + (r * kU + u) * 1024 + 16 * lane);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[r][g] = mfma16(aq[b & 1][u][g], unpack_scaled(bw, g),
                                       b == 0 && u == 0 ? v4i{0, 0, 0, 0} : acc[r][g]);
            }
        }
    }, std::make_integer_sequence<int, NB>{});

    // 5. Sum the fields, then the ks waves of each tile group.
    //    D(i, j) lives in lane j + 16*(i/4), register i%4.  Useful lanes:
    //    [0, 8) and [16, 24) (even chunks, row j, tokens 4*(lane/16) + c) and
    //    lane + 40 (odd chunks, same row and tokens).
    const int l = lane;
    auto store = [&](int r, const v4i &t) {
        const int n = n0 + r * kTileRows + (l & 7);
        if (n >= N) return;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = 4 * (l >> 4) + c;
            if (m < M) {
                const int mm = m < FM ? m : 0;
                const int qs = FM > 0 ? (qpart_sh[mm][0] + qpart_sh[mm][1]) +
                                            (qpart_sh[mm][2] + qpart_sh[mm][3])
                                      : qs_pre[c];
                const int v = t[c] - qs;
                if (OUT_Y) {
                    const float iv = FM > 0 ? inv_sh[m < FM ? m : 0] : iv_pre[c];
                    store_out(reinterpret_cast<IO *>(P.y), (size_t)m * N + n,
                              (float)v * (P.w_scale / iv));
                } else {
                    P.acc[(size_t)m * N + n] = v;
                }
            }
        }
    };
    if (ks == 1) {
        // Each wave owns whole tiles (ks is uniform over the workgroup):
        // the parity halves meet by a lane permute, no LDS, no barrier.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const v4i s4 = field_sum(acc[r]);
            v4i t;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                t[c] = s4[c] + __builtin_amdgcn_ds_bpermute(((l + 40) & 63) << 2, s4[c]);
            if ((l & 8) == 0 && l < 24) store(r, t);
        }
        return;
    }
    // ks > 1: the partial tiles go to each wave's first weight buffer, no
    // longer needed, and the first wave of each group sums them.
    v4i *part = reinterpret_cast<v4i *>(&w0[0][0]);  // [W][SZ / 16] v4i, R * 64 used
    constexpr int PS = SZ / 16;
#pragma unroll
    for (int r = 0; r < R; ++r)
        part[wid * PS + r * 64 + lane] = field_sum(acc[r]);
    lds_barrier();
    if (kp == 0 && (l & 8) == 0 && l < 24) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int o = r * 64 + l;
            v4i t = part[wid * PS + o] + part[wid * PS + o + 40];
            for (int w = 1; w < ks; ++w) t += part[(wid + w) * PS + o] + part[(wid + w) * PS + o + 40];
            store(r, t);
        }
    }
}

// Rolling form of the same contraction, for problem sets larger than the
// device holds at once (the 70B FFN matrices at one token).  The one-shot
// kernel issues all of a wave's loads up front; once the compute unit's
// memory pipeline is full, a wave stalls at the issue of its remaining loads
// and cannot contract what has arrived, and the quantisation's barriers make
// every wave of the workgroup wait for the slowest issuer -- so the
// contraction only starts near the end of the stream.  Here each wave keeps
// a ring of ND batches in registers: it issues ND batches before the
// quantisation, then contracts batch b and issues batch b + ND into its
// slot, so no issue waits long and the contraction keeps pace with the
// stream.  A wave covers its tile group's K share (ks waves per tile group)
// in any number of batches; the batch count is padded to a multiple of ND
// with range-checked loads that read nothing, so the loop body is the same
// every time and the compiler's load counts stay exact.  Launch: one
// workgroup per tile-group set, W = 16 waves (one per CU by registers).
template <int ND, int R, bool OUT_Y, int FM, int SQ, typename IO = float, int W = 16,
          bool GLU = false>
__global__ __launch_bounds__(64 * W) void gemv_roll_kernel(int b0, int b1, int b2, int b3, int b4,
                                                        int b5, int b6, int b7, ShotBatch B) {
    static_assert(ND >= 1 && ND <= 4, "ring depth");
    static_assert(R == 1 || R == 2, "tiles per wave");
    static_assert(W == 4 || W == 8 || W == 16, "waves per workgroup");
    static_assert(kU == 2, "shift forms below assume kU == 2");
    static_assert(FM == 0 || (FM == 1 && W == 16), "fused: one token, 16 waves");
    static_assert(!GLU || FM == 1, "the gated input is fused");
    static_assert(SQ == 1 || SQ == 2 || SQ == 4 || SQ == 8, "row segment");
    constexpr int LW = W == 16 ? 4 : W == 8 ? 3 : 2;
    extern __shared__ __align__(16) int8_t q_lds[];
    __shared__ float red[20];
    __shared__ float chain_sh[FM > 0 ? 256 : 1];
    __shared__ float inv_sh[1];
    __shared__ int qpart_sh[16];
    __shared__ __align__(16) v4i part[W][R * 64];  // partial tiles when ks > 1

    (void)b0;
    const int bx = (int)blockIdx.x;
    const int pi = (bx >= b1) + (bx >= b2) + (bx >= b3) + (bx >= b4) + (bx >= b5) + (bx >= b6) +
                   (bx >= b7);
    const ShotBatch *Bk = reinterpret_cast<const ShotBatch *>(
        (const char *)__builtin_amdgcn_kernarg_segment_ptr() + 8 * sizeof(int));
    const ShotProblem P = Bk->p[pi];
    asm volatile("" ::"s"(P.q), "s"(P.inv), "s"(P.qsum), "s"(P.x), "s"(P.gamma), "s"(P.q_out),
                 "s"(P.inv_out), "s"(P.qsum_out), "s"(P.packed), "s"(P.y), "s"(P.acc), "s"(P.eps),
                 "s"(P.w_scale), "s"(P.M), "s"(P.K), "s"(P.N), "s"(P.wg_begin), "s"(P.ks_log));
    if constexpr (GLU) asm volatile("" ::"s"(P.u));
    const int M = P.M, K = P.K, N = P.N;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r8 = lane & 7;
    const int ch = lane >> 3;
    const uint32_t rowbytes = (uint32_t)K / 4;
    const int nsteps = (int)((rowbytes + kStep - 1) / kStep);
    const int kl = P.ks_log;
    const int ks = 1 << kl;
    const int sg = wid >> kl, kp = wid & (ks - 1);
    const int nb = (nsteps + ks * kU - 1) >> (kl + 1);
    const int nbp = (nb + ND - 1) / ND * ND;  // padded to whole rounds of the ring
    const int st = bx - P.wg_begin;
    const int tg = (st << (LW - kl)) + sg;
    const int n0 = tg * kTileRows * R;
    const int rows = max(0, min(kTileRows * R, N - n0));
    const auto rw = make_rsrc(P.packed + (size_t)min(n0, N) * rowbytes, (uint32_t)rows * rowbytes);

    // Batch b of this wave into a ring slot (past the wave's batches:
    // range-checked to read nothing).
    v4i ring[ND][R][kU];
    auto issue = [&](v4i(&slot)[R][kU], int b) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int s = b * ks * kU + kp * kU + u;
                const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
                const bool kv = b < nb && s < nsteps && cb < rowbytes;
                slot[r][u] = buf_load16(rw, kv ? (uint32_t)(r * kTileRows + r8) * rowbytes + cb : kOOB);
            }
        }
    };
    auto prologue = [&] {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < ND; ++j) issue(ring[j], j);
        __builtin_amdgcn_sched_barrier(0);
    };

    int qs_pre[4];
    float iv_pre[4];
    if constexpr (FM == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = min(4 * (lane >> 4) + c, M - 1);
            qs_pre[c] = P.qsum[m];
            iv_pre[c] = OUT_Y ? P.inv[m] : 1.0f;
        }
        // The activation block goes ahead of every weight load of the
        // workgroup (barrier), the ring's first batches behind it.
        const uint32_t qbytes = (uint32_t)(M * K);
        const auto rq = make_rsrc(P.q, qbytes);
        for (uint32_t c = (uint32_t)wid * 1024u; c < qbytes; c += W * 1024u)
            buf_load16_lds(rq, q_lds + c, c + 16u * lane, 0);
        __builtin_amdgcn_s_barrier();
        prologue();
        wait_vmcnt<ND * R * kU>();
        lds_barrier();
    } else if constexpr (SQ <= 2) {
        // Rows of up to 8192: waves 0..3 quantise the row in the 256-thread
        // block form (its reductions meeting on an LDS counter among the
        // four), the other waves issue their rings at once, behind the
        // barrier that puts the x / gamma loads first, and the quantising
        // waves issue theirs once q is published, so that their issue
        // stalls never hold the quantisation up.
        __shared__ int spin_sh;
        if (tid < 16) qpart_sh[tid] = 0;  // waves 4..15 add no partial sum
        if (tid == 0) spin_sh = 0;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): visible past the barrier below
        QuadSpin meet{&spin_sh, 0};
        if (wid < 4) {
            ShotRowSink sink{q_lds, inv_sh, qpart_sh, st == 0 ? P.q_out : nullptr, P.inv_out};
            block_act_quant_row<8, false, true, GLU, float>(P.x, P.gamma, P.eps, K, red, sink,
                                                            [] {}, P.u, &meet);
        } else {
            __builtin_amdgcn_s_barrier();  // behind the x / gamma loads
            prologue();
        }
        lds_barrier();
        if (wid < 4) prologue();
        if (st == 0 && tid == 0) {
            int t = 0;
            for (int w = 0; w < 16; ++w) t += qpart_sh[w];
            P.qsum_out[0] = t;
        }
    } else {
        // The whole row of x and gamma over all 16 waves (one round trip,
        // ahead of every weight load of the workgroup), then the ring's
        // first batches; the quantisation runs while they stream in.
        wide_act_quant_row<SQ, GLU>(P.x, P.gamma, P.eps, K, red, chain_sh, q_lds,
                                    st == 0 ? P.q_out : nullptr, inv_sh, P.inv_out, qpart_sh,
                                    prologue, P.u);
        lds_barrier();
        if (st == 0 && tid == 0) {
            int t = 0;
            for (int w = 0; w < 16; ++w) t += qpart_sh[w];
            P.qsum_out[0] = t;
        }
    }

    // Contraction: batch b from ring slot b % ND, then batch b + ND into it.
    const int qrow = min(r8, M - 1) * K;
    v4i acc[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[r][g] = v4i{0, 0, 0, 0};
    for (int bb = 0; bb < nbp; bb += ND) {
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            const int b = bb + j;
            if (b < nb) {  // the padding batches hold zeros: no contraction
                v4i aq[kU][4];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int s = b * ks * kU + kp * kU + u;
                    const uint32_t cb = (uint32_t)s * kStep + 16u * ch;
                    const bool kv = s < nsteps && cb < rowbytes;
                    const int kb =
                        kv ? (int)(cb / 32) * kBlockWeights + 16 * (int)((cb / 16) & 1) : 0;
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        aq[u][g] = *reinterpret_cast<const v4i *>(q_lds + qrow + kb + 32 * g);
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int u = 0; u < kU; ++u)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            acc[r][g] =
                                mfma16(aq[u][g], unpack_scaled(ring[j][r][u], g), acc[r][g]);
            }
            issue(ring[j], b + ND);
        }
    }

    // Fields, then the ks waves of each tile group (as in the one-shot form).
    const int l = lane;
    auto store = [&](int r, const v4i &t) {
        const int n = n0 + r * kTileRows + (l & 7);
        if (n >= N) return;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = 4 * (l >> 4) + c;
            if (m < M) {
                int qs = qs_pre[c];
                if constexpr (FM > 0) {
                    qs = 0;
                    for (int w = 0; w < 16; ++w) qs += qpart_sh[w];
                }
                const int v = t[c] - qs;
                if (OUT_Y) {
                    const float iv = FM > 0 ? inv_sh[0] : iv_pre[c];
                    store_out(reinterpret_cast<IO *>(P.y), (size_t)m * N + n,
                              (float)v * (P.w_scale / iv));
                } else {
                    P.acc[(size_t)m * N + n] = v;
                }
            }
        }
    };
    if (ks == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const v4i s4 = field_sum(acc[r]);
            v4i t;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                t[c] = s4[c] + __builtin_amdgcn_ds_bpermute(((l + 40) & 63) << 2, s4[c]);
            if ((l & 8) == 0 && l < 24) store(r, t);
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) part[wid][r * 64 + lane] = field_sum(acc[r]);
    lds_barrier();
    if (kp == 0 && (l & 8) == 0 && l < 24) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int o = r * 64 + l;
            v4i t = part[wid][o] + part[wid][o + 40];
            for (int w = 1; w < ks; ++w) t += part[wid + w][o] + part[wid + w][o + 40];
            store(r, t);
        }
    }
}

// Smallest K split (waves per tile group) that fits a wave's share of a
// row into NB batches, or 0.
int shot_ks(int64_t K, int nbmax) {
    const int64_t nsteps = (K / 4 + kStep - 1) / kStep;
    for (int ks = 1; ks <= kMaxKs; ks *= 2)
        if ((nsteps + ks * kU - 1) / (ks * kU) <= nbmax) return ks;
    return 0;
}

// Fills the batch: each problem's K split and first workgroup (begin[i];
// INT_MAX past the last problem).  Returns the grid size; *qmax receives the
// largest activation block (bytes).
int64_t fill_batch(ShotBatch &B, int *begin, int count, int nb, int R, int W, const int64_t *M,
                   const int64_t *K, const int64_t *N, int64_t *qmax) {
    int64_t gx = 0;
    *qmax = 0;
    for (int i = 0; i < count; ++i) {
        const int ks = shot_ks(K[i], nb);
        const int64_t ntg = (N[i] + kTileRows * R - 1) / (kTileRows * R);
        const int64_t nset = (ntg + W / ks - 1) / (W / ks);
        ShotProblem &P = B.p[i];
        P.M = (int)M[i];
        P.K = (int)K[i];
        P.N = (int)N[i];
        P.ks_log = ks == 1 ? 0 : ks == 2 ? 1 : 2;
        P.wg_begin = (int)gx;
        begin[i] = (int)gx;
        gx += nset;
        *qmax = std::max<int64_t>(*qmax, M[i] * K[i]);
    }
    for (int i = count; i < kMaxShotBatch; ++i) begin[i] = INT_MAX;
    return gx;
}

template <class Kernel>
hipError_t launch_batch(Kernel kern, int W, const ShotBatch &B, const int *b, int64_t gx,
                        int64_t qmax, hipStream_t s) {
    const size_t lds = (size_t)((qmax + 1023) / 1024 * 1024);
    if (gx < 1 || gx > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)gx), dim3(64 * W), lds, s, b[0], b[1], b[2], b[3], b[4],
                       b[5], b[6], b[7], B);
    return hipGetLastError();
}

// Launch shapes: weight batches per wave (NB) x tiles per wave (R) x waves
// per workgroup (W).  A workgroup holds NB * R * W * 2 KB of weights in LDS.
struct ShotShape {
    int nb, R;
    int occupancy;  // workgroups per CU that the registers allow
    int w;
};
constexpr ShotShape kShotShapes[] = {{3, 1, 4, 4}, {4, 1, 4, 4}, {8, 1, 4, 4}, {3, 2, 3, 4},
                                     {4, 2, 3, 4}, {2, 2, 1, 8}, {3, 2, 1, 8}, {3, 1, 1, 16}};
constexpr int kNumShotShapes = sizeof(kShotShapes) / sizeof(kShotShapes[0]);
static_assert(kNumShotShapes == kShotShapeCount, "shape count the variant numbering uses");

}  // namespace

// Compute units of the current device, looked up once per device (the
// launch-shape choice runs on every call).  Devices beyond the table are
// queried each time.
int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];  // 0: not looked up yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        return 256;
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

namespace {

// Launch-shape choice.  A shape costs (in this order): the rounds of
// workgroups the device needs to hold them all (resident workgroups per CU
// from LDS and registers; more than one round leaves the later workgroups'
// loads waiting for earlier ones to finish); then a score: the share of the
// allocated weight LDS that stays unused (rows whose K share is shorter
// than NB batches), weighted by bytes, plus small measured preferences.
// With the quantisation fused in, two tiles per wave beat one (half the
// workgroups repeat the quantisation) unless the device would be left
// underfilled; over q from global memory one tile per wave is the faster
// (measured on MI355X, M = 1..4, K = 2560..8192: up to 1.4x).  One
// workgroup per CU costs extra.
// One token with the quantisation fused in (the decode case) takes, after
// rounds, an estimate of the launch time instead of that score, and is the
// only case that considers the 8- and 16-wave shapes (one_token_cost; not
// taken with the gated FFN input, `wide` false).
// *rounds_out receives the chosen shape's rounds.
// Estimated time (us) of a one-round fused launch for one token, a linear
// model fitted to the measured times of every shape on ten decode problem
// sets (M = 1, K = 2048..8192, one to seven BitLinears, 1.7 to 37 MB;
// MI355X, two runs averaged; rms error 0.3 us).  A CU that holds c
// workgroups streams c times the largest workgroup's weight bytes and runs
// c quantisation chains of up to max K elements; splitting a row's K over 2
// or 4 waves costs the partial-sum reduction and shorter streams; a launch
// of fewer workgroups than CUs runs faster than those terms say; the rest
// is a fixed cost per shape (lower for the 8- and 16-wave workgroups: one
// quantisation per CU, its four waves meeting among themselves while the
// others issue their weights).  It picks the fastest shape in every set;
// fitted with each set left out in turn, its picks sum to within 0.7 % of
// the fastest shapes'.
constexpr double kOneTokenBase[kShotShapeCount] = {3.52, 3.74, 4.69, 4.19,
                                                   4.52, 3.76, 3.49, 3.20};
double one_token_cost(int v, const int64_t *K, const int64_t *N, int count, int cus) {
    const ShotShape &h = kShotShapes[v];
    int64_t wgs = 0, kmax = 0;
    double wg_bytes = 0.0;
    int ksmax = 1;
    for (int i = 0; i < count; ++i) {
        const int ks = shot_ks(K[i], h.nb);
        const int slots = h.w / ks;
        const int64_t ntg = (N[i] + kTileRows * h.R - 1) / (kTileRows * h.R);
        wgs += (ntg + slots - 1) / slots;
        wg_bytes = std::max(wg_bytes, (double)slots * kTileRows * h.R * (double)(K[i] / 4));
        kmax = std::max<int64_t>(kmax, K[i]);
        ksmax = std::max(ksmax, ks);
    }
    const double c = (double)((wgs + cus - 1) / cus);
    const double under = std::max(0.0, 1.0 - (double)wgs / cus);
    return 0.035 * c * wg_bytes / 1024.0 + 0.098 * c * (double)kmax / 1024.0 +
           (ksmax == 4 ? 0.50 : ksmax == 2 ? 0.37 : 0.0) - 0.89 * under + kOneTokenBase[v];
}

int pick_shape(const int64_t *M, const int64_t *K, const int64_t *N, int count, int pref,
               int64_t *rounds_out, bool fused, bool wide = true) {
    auto fits = [&](int nb) {
        for (int i = 0; i < count; ++i)
            if (shot_ks(K[i], nb) == 0) return false;
        return true;
    };
    int64_t qmax = 0;
    for (int i = 0; i < count; ++i) qmax = std::max<int64_t>(qmax, M[i] * K[i]);
    const int64_t q = (qmax + 1023) / 1024 * 1024;
    const int cus = device_cus();
    auto wgs_of = [&](const ShotShape &h) -> int64_t {
        int64_t wgs = 0;
        for (int i = 0; i < count; ++i) {
            const int ks = shot_ks(K[i], h.nb);
            const int64_t ntg = (N[i] + kTileRows * h.R - 1) / (kTileRows * h.R);
            wgs += (ntg + h.w / ks - 1) / (h.w / ks);
        }
        return wgs;
    };
    auto rounds_of = [&](const ShotShape &h) -> int64_t {
        const int64_t wgs = wgs_of(h);
        const int64_t lds = (int64_t)h.nb * h.R * h.w * 2048 + q + 256;
        const int64_t per_cu = std::min<int64_t>(h.occupancy, (160 * 1024) / lds);
        return per_cu < 1 ? INT64_MAX : (wgs + per_cu * cus - 1) / (per_cu * cus);
    };
    // A requested shape is taken when every problem fits it and its LDS
    // (weights and activation block) fits a CU.
    if (pref >= 1 && pref <= kNumShotShapes && fits(kShotShapes[pref - 1].nb) &&
        rounds_of(kShotShapes[pref - 1]) != INT64_MAX) {
        *rounds_out = rounds_of(kShotShapes[pref - 1]);
        return pref - 1;
    }
    bool one_token = fused && wide;
    for (int i = 0; i < count; ++i) one_token = one_token && M[i] == 1;
    int best = -1;
    int64_t best_rounds = 0;
    double best_score = 0.0;
    for (int v = 0; v < kNumShotShapes; ++v) {
        const ShotShape &h = kShotShapes[v];
        if (!fits(h.nb) || (h.w != 4 && !one_token)) continue;
        const int64_t rounds = rounds_of(h);
        if (rounds == INT64_MAX) continue;
        if (one_token) {
            const double est = one_token_cost(v, K, N, count, cus);
            if (best < 0 || rounds < best_rounds || (rounds == best_rounds && est < best_score)) {
                best = v;
                best_rounds = rounds;
                best_score = est;
            }
            continue;
        }
        double used = 0.0, total = 0.0;
        for (int i = 0; i < count; ++i) {
            const int64_t nsteps = (K[i] / 4 + kStep - 1) / kStep;
            const int ks = shot_ks(K[i], h.nb);
            const double bytes = (double)N[i] * (double)(K[i] / 4);
            used += bytes * ((double)nsteps / ks) / (h.nb * kU);
            total += bytes;
        }
        const int64_t lds = (int64_t)h.nb * h.R * h.w * 2048 + q + 256;
        const int64_t per_cu = std::min<int64_t>(h.occupancy, (160 * 1024) / lds);
        double score = 100.0 * (1.0 - used / total);
        if (fused)
            score += h.R == 1 ? 10.0 : 0.0;
        else
            score += h.R == 2 ? 10.0 : 0.0;
        // Fewer workgroups than CUs leave CUs without weights to stream:
        // with the quantisation fused in this outweighs the tile
        // preference (one BitLinear of N = 2560 at K = 6912: one tile per
        // wave 5.7 us against two tiles 7.2 us, measured).
        if (fused) score += 60.0 * std::max(0.0, 1.0 - (double)wgs_of(h) / cus);
        score += per_cu == 1 ? 20.0 : 0.0;
        // Over q from global memory: more resident workgroups per CU keep
        // more weight loads in flight.
        if (!fused) score += 5.0 * (double)(4 - std::min<int64_t>(per_cu, 4));
        // Fused: a later round repeats the quantisation chain, so rounds come
        // first.  Over q from global memory the score comes first: more
        // resident waves per CU beat fewer rounds (N = 28672, K = 8192:
        // 4 batches x 1 tile over 3 rounds 12.4 us, 8 x 1 over 2 rounds
        // 15.6 us, measured).
        const bool better =
            fused ? (rounds < best_rounds || (rounds == best_rounds && score < best_score))
                  : (score < best_score || (score == best_score && rounds < best_rounds));
        if (best < 0 || better) {
            best = v;
            best_rounds = rounds;
            best_score = score;
        }
    }
    *rounds_out = best_rounds;
    return best;
}

template <int NB, int R, int W, bool OUT_Y, typename IO>
hipError_t launch_shot_nb(const ShotDecode *d, int count, hipStream_t s) {
    ShotBatch B{};
    int64_t M[kMaxShotBatch], K[kMaxShotBatch], N[kMaxShotBatch], qmax;
    for (int i = 0; i < count; ++i) {
        M[i] = d[i].M;
        K[i] = d[i].K;
        N[i] = d[i].N;
        ShotProblem &P = B.p[i];
        P.q = d[i].q;
        P.inv = d[i].inv;
        P.qsum = d[i].qsum;
        P.packed = d[i].packed;
        P.y = d[i].y;
        P.acc = d[i].acc;
        P.w_scale = d[i].w_scale;
    }
    int begin[kMaxShotBatch];
    const int64_t gx = fill_batch(B, begin, count, NB, R, W, M, K, N, &qmax);
    return launch_batch(gemv_shot_kernel<NB, R, OUT_Y, 0, 1, false, false, IO, W>, W, B, begin, gx,
                        qmax, s);
}

template <int NB, int R, int W, int FM, int CH, bool LONG, bool GLU, typename IO>
hipError_t launch_shot_fused_nb(const FusedDecode *d, int count, hipStream_t s) {
    ShotBatch B{};
    int64_t M[kMaxShotBatch], K[kMaxShotBatch], N[kMaxShotBatch], qmax;
    for (int i = 0; i < count; ++i) {
        M[i] = d[i].M;
        K[i] = d[i].K;
        N[i] = d[i].N;
        ShotProblem &P = B.p[i];
        P.x = d[i].x;
        P.gamma = d[i].gamma;
        P.q_out = d[i].q;
        P.inv_out = d[i].inv;
        P.qsum_out = d[i].qsum;
        P.packed = d[i].packed;
        P.y = d[i].y;
        P.eps = d[i].eps;
        P.w_scale = d[i].w_scale;
        P.u = d[i].u;
    }
    int begin[kMaxShotBatch];
    const int64_t gx = fill_batch(B, begin, count, NB, R, W, M, K, N, &qmax);
    return launch_batch(gemv_shot_kernel<NB, R, true, FM, CH, LONG, GLU, IO, W>, W, B, begin, gx,
                        qmax, s);
}

#define BL_SHOT_SHAPES(CALL)                                                   \
    switch (v) {                                                               \
        case 0: return CALL(3, 1, 4);                                          \
        case 1: return CALL(4, 1, 4);                                          \
        case 2: return CALL(8, 1, 4);                                          \
        case 3: return CALL(3, 2, 4);                                          \
        case 4: return CALL(4, 2, 4);                                          \
        case 5: return CALL(2, 2, 8);                                          \
        case 6: return CALL(3, 2, 8);                                          \
        case 7: return CALL(3, 1, 16);                                         \
        default: return hipErrorInvalidValue;                                  \
    }

template <int FM, int CH, bool LONG, bool GLU = false, typename IO = float>
hipError_t launch_fused_ch(const FusedDecode *d, int count, int v, hipStream_t s) {
#define BL_F(NB_, R_, W_) launch_shot_fused_nb<NB_, R_, W_, FM, CH, LONG, GLU, IO>(d, count, s)
    BL_SHOT_SHAPES(BL_F)
#undef BL_F
}

template <bool OUT_Y, typename IO = float>
hipError_t launch_sep(const ShotDecode *d, int count, int v, hipStream_t s) {
#define BL_S(NB_, R_, W_) launch_shot_nb<NB_, R_, W_, OUT_Y, IO>(d, count, s)
    BL_SHOT_SHAPES(BL_S)
#undef BL_S
}

}  // namespace

int shot_num_shapes() { return kNumShotShapes; }

int64_t shot_rounds(const int64_t *M, const int64_t *K, const int64_t *N, int count, bool fused,
                    bool glu) {
    for (int i = 0; i < count; ++i)
        if (!shot_supported(M[i], K[i])) return INT64_MAX;
    int64_t rounds;
    return pick_shape(M, K, N, count, 0, &rounds, fused, !glu) < 0 ? INT64_MAX : rounds;
}

bool shot_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= kMaxShotM && M * K <= kShotMaxQ && shot_ks(K, 8) != 0;
}

bool shot_fused_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= kFuseMaxM && M * K <= kShotFusedMaxQ && shot_ks(K, 8) != 0;
}

// The 16-wave shape: four quads quantise up to four rows side by side.
// Measured on MI355X with the quantisation fused in, against the separate
// quantisation + contraction pair (us, M = 2 / 3): decoder layer 8.1 / 9.6
// against 10.5 / 11.8; K = N = 8192 8.4 / 10.2 against 9.7 / 10.0; three
// 4096 x 4096 BitLinears 7.0 / 8.4 against 8.7 / 9.0.  At M = 4 every wave
// quantises and all weights go out after it: slower on two of the three
// (12.1 against 10.5 us at K = N = 8192), so the pair keeps M = 4.  The
// 8-wave shapes measured slower than this one on all three.
constexpr int kFewTokenShape = 7;
static_assert(kShotShapes[kFewTokenShape].w == 16, "four quads");
static_assert(kFewFusedShapeVariant == kFewTokenShape + 1, "shape numbering of launch_gemv_shot_fused");

bool few_fused_one_round(const int64_t *M, const int64_t *K, const int64_t *N, int count) {
    if (count < 1 || count > kMaxShotBatch) return false;
    for (int i = 0; i < count; ++i)
        if (M[i] < 1 || M[i] > kFewFusedMaxM || K[i] > 8192 || !shot_fused_supported(M[i], K[i]))
            return false;
    int64_t rounds = 0;
    return pick_shape(M, K, N, count, kFewTokenShape + 1, &rounds, true) == kFewTokenShape &&
           rounds == 1;
}

hipError_t launch_gemv_shot(const ShotDecode *d, int count, int shape, hipStream_t s) {
    if (count < 1 || count > kMaxShotBatch) return hipErrorInvalidValue;
    const bool y = d[0].y != nullptr;
    const int io = d[0].io;
    int64_t M[kMaxShotBatch], K[kMaxShotBatch], N[kMaxShotBatch];
    for (int i = 0; i < count; ++i) {
        if (!shot_supported(d[i].M, d[i].K) || (d[i].y != nullptr) != y || d[i].io != io ||
            (io != kIoF32 && !y))
            return hipErrorInvalidValue;
        M[i] = d[i].M;
        K[i] = d[i].K;
        N[i] = d[i].N;
    }
    int64_t rounds;
    const int v = pick_shape(M, K, N, count, shape, &rounds, false);
    if (!y) return launch_sep<false>(d, count, v, s);
    if (io == kIoBf16) return launch_sep<true, bf16_t>(d, count, v, s);
    if (io == kIoF16) return launch_sep<true, _Float16>(d, count, v, s);
    return launch_sep<true>(d, count, v, s);
}

hipError_t launch_gemv_shot_fused(const FusedDecode *d_in, int count, int shape, hipStream_t s) {
    if (count < 1 || count > kMaxShotBatch) return hipErrorInvalidValue;
    // Problems in order of decreasing K (stable): workgroups are dispatched
    // in index order, so the longest quantisation chains start first.
    FusedDecode ord[kMaxShotBatch];
    for (int i = 0; i < count; ++i) ord[i] = d_in[i];
    std::stable_sort(ord, ord + count,
                     [](const FusedDecode &a, const FusedDecode &b) { return a.K > b.K; });
    const FusedDecode *d = ord;
    int64_t M[kMaxShotBatch], K[kMaxShotBatch], N[kMaxShotBatch], kmax = 0, mmax = 0;
    const bool glu = d[0].u != nullptr;
    const int io = d[0].io;
    for (int i = 0; i < count; ++i) {
        if (!shot_fused_supported(d[i].M, d[i].K) || !d[i].y) return hipErrorInvalidValue;
        if ((d[i].u != nullptr) != glu || (glu && d[i].M != 1)) return hipErrorInvalidValue;
        // half-precision I/O: one token, rows held in registers, one type
        if (d[i].io != io || (io != kIoF32 && (glu || d[i].M != 1 || d[i].K > 8192)))
            return hipErrorInvalidValue;
        M[i] = d[i].M;
        K[i] = d[i].K;
        N[i] = d[i].N;
        kmax = std::max<int64_t>(kmax, d[i].K);
        mmax = std::max<int64_t>(mmax, d[i].M);
    }
    int64_t rounds;
    const int v = pick_shape(M, K, N, count, shape, &rounds, true, !glu);
    // One token everywhere (the decode case): the kernel that normalises a
    // single row, whose code is a quarter of the general one's.
    if (io == kIoBf16) {
        if (kmax <= 4096) return launch_fused_ch<1, 4, false, false, bf16_t>(d, count, v, s);
        return launch_fused_ch<1, 8, false, false, bf16_t>(d, count, v, s);
    }
    if (io == kIoF16) {
        if (kmax <= 4096) return launch_fused_ch<1, 4, false, false, _Float16>(d, count, v, s);
        return launch_fused_ch<1, 8, false, false, _Float16>(d, count, v, s);
    }
    if (glu) {
        if (kmax <= 4096) return launch_fused_ch<1, 4, false, true>(d, count, v, s);
        if (kmax <= 8192) return launch_fused_ch<1, 8, false, true>(d, count, v, s);
        return launch_fused_ch<1, 8, true, true>(d, count, v, s);
    }
    if (mmax == 1) {
        if (kmax <= 4096) return launch_fused_ch<1, 4, false>(d, count, v, s);
        if (kmax <= 8192) return launch_fused_ch<1, 8, false>(d, count, v, s);
        return launch_fused_ch<1, 8, true>(d, count, v, s);
    }
    if (kmax <= 4096) return launch_fused_ch<kFuseMaxM, 4, false>(d, count, v, s);
    if (kmax <= 8192) return launch_fused_ch<kFuseMaxM, 8, false>(d, count, v, s);
    return launch_fused_ch<kFuseMaxM, 8, true>(d, count, v, s);
}

#undef BL_SHOT_SHAPES

namespace {

constexpr int kRollW = 16;  // waves per workgroup of the rolling form
constexpr int kRollND = 3;  // ring depth (batches per wave in flight)

// K split of each problem for the rolling form.  Workgroups should carry
// about the same bytes (a workgroup's rows are 16 / ks tile groups of K / 4
// bytes each): each problem first splits until its workgroups carry at most
// 1.5 times those of the shortest rows' (rows of 28672 beside rows of 8192
// take 4 waves per tile group).  Then, while the launch has fewer
// workgroups than about the compute units, the problem whose workgroups
// carry the most bytes splits further -- up to all 16 waves on one tile
// group, each keeping at least two 128-byte steps of the row.  Fills ks_log,
// wg_begin and M/K/N; returns the grid.
int64_t fill_roll(ShotBatch &B, int *begin, int count, const int64_t *M, const int64_t *K,
                  const int64_t *N, int64_t *qmax) {
    const int cus = device_cus();
    int ks[kMaxShotBatch];
    int64_t ntg[kMaxShotBatch];
    auto wgs_of = [&](int i) { return (ntg[i] + kRollW / ks[i] - 1) / (kRollW / ks[i]); };
    auto per_wg = [&](int i) { return (double)(kRollW / ks[i]) * kTileRows * (double)(K[i] / 4); };
    auto can_split = [&](int i) {
        return ks[i] < kRollW && (K[i] / 4 + kStep - 1) / kStep >= 4 * ks[i];
    };
    int64_t kmin = INT64_MAX;
    *qmax = 0;
    for (int i = 0; i < count; ++i) {
        ks[i] = 1;
        ntg[i] = (N[i] + kTileRows - 1) / kTileRows;
        kmin = std::min(kmin, K[i]);
        *qmax = std::max<int64_t>(*qmax, M[i] * K[i]);
    }
    const double floor_bytes = (double)kRollW * kTileRows * (double)(kmin / 4);
    int64_t total = 0;
    for (int i = 0; i < count; ++i) {
        while (can_split(i) && per_wg(i) > 1.5 * floor_bytes) ks[i] *= 2;
        total += wgs_of(i);
    }
    while (total * 8 < (int64_t)cus * 7) {
        int best = -1;
        for (int i = 0; i < count; ++i)
            if (can_split(i) && (best < 0 || per_wg(i) > per_wg(best))) best = i;
        if (best < 0) break;
        total -= wgs_of(best);
        ks[best] *= 2;
        total += wgs_of(best);
    }
    int64_t gx = 0;
    for (int i = 0; i < count; ++i) {
        ShotProblem &P = B.p[i];
        P.M = (int)M[i];
        P.K = (int)K[i];
        P.N = (int)N[i];
        P.ks_log = ks[i] == 1 ? 0 : ks[i] == 2 ? 1 : ks[i] == 4 ? 2 : ks[i] == 8 ? 3 : 4;
        P.wg_begin = (int)gx;
        begin[i] = (int)gx;
        gx += wgs_of(i);
    }
    for (int i = count; i < kMaxShotBatch; ++i) begin[i] = INT_MAX;
    return gx;
}

template <bool OUT_Y>
hipError_t launch_roll_sep(const ShotDecode *d, int count, hipStream_t s) {
    ShotBatch B{};
    int64_t M[kMaxShotBatch], K[kMaxShotBatch], N[kMaxShotBatch], qmax;
    for (int i = 0; i < count; ++i) {
        M[i] = d[i].M;
        K[i] = d[i].K;
        N[i] = d[i].N;
        ShotProblem &P = B.p[i];
        P.q = d[i].q;
        P.inv = d[i].inv;
        P.qsum = d[i].qsum;
        P.packed = d[i].packed;
        P.y = d[i].y;
        P.acc = d[i].acc;
        P.w_scale = d[i].w_scale;
    }
    int begin[kMaxShotBatch];
    const int64_t gx = fill_roll(B, begin, count, M, K, N, &qmax);
    return launch_batch(gemv_roll_kernel<kRollND, 1, OUT_Y, 0, 1, float, kRollW>, kRollW, B,
                        begin, gx, qmax, s);
}

template <int SQ, bool GLU>
hipError_t launch_roll_fused(const FusedDecode *d, int count, hipStream_t s) {
    ShotBatch B{};
    int64_t M[kMaxShotBatch], K[kMaxShotBatch], N[kMaxShotBatch], qmax;
    for (int i = 0; i < count; ++i) {
        M[i] = d[i].M;
        K[i] = d[i].K;
        N[i] = d[i].N;
        ShotProblem &P = B.p[i];
        P.x = d[i].x;
        P.gamma = d[i].gamma;
        P.q_out = d[i].q;
        P.inv_out = d[i].inv;
        P.qsum_out = d[i].qsum;
        P.packed = d[i].packed;
        P.y = d[i].y;
        P.eps = d[i].eps;
        P.w_scale = d[i].w_scale;
        P.u = d[i].u;
    }
    int begin[kMaxShotBatch];
    const int64_t gx = fill_roll(B, begin, count, M, K, N, &qmax);
    return launch_batch(gemv_roll_kernel<kRollND, 1, true, 1, SQ, float, kRollW, GLU>, kRollW, B,
                        begin, gx, qmax, s);
}

}  // namespace

bool roll_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= kMaxShotM && M * K <= kShotMaxQ && K % kBlockWeights == 0;
}

hipError_t launch_gemv_roll(const ShotDecode *d, int count, hipStream_t s) {
    if (count < 1 || count > kMaxShotBatch) return hipErrorInvalidValue;
    const bool y = d[0].y != nullptr;
    for (int i = 0; i < count; ++i)
        if (!roll_supported(d[i].M, d[i].K) || (d[i].y != nullptr) != y || d[i].io != kIoF32)
            return hipErrorInvalidValue;
    return y ? launch_roll_sep<true>(d, count, s) : launch_roll_sep<false>(d, count, s);
}

bool roll_fused_supported(int64_t M, int64_t K) {
    return M == 1 && K <= kShotFusedMaxQ && K % kBlockWeights == 0;
}

hipError_t launch_gemv_roll_fused(const FusedDecode *d, int count, hipStream_t s) {
    if (count < 1 || count > kMaxShotBatch) return hipErrorInvalidValue;
    int64_t kmax = 0;
    const bool glu = d[0].u != nullptr;
    for (int i = 0; i < count; ++i) {
        if (!roll_fused_supported(d[i].M, d[i].K) || !d[i].y || (d[i].u != nullptr) != glu ||
            d[i].io != kIoF32)
            return hipErrorInvalidValue;
        kmax = std::max<int64_t>(kmax, d[i].K);
    }
    // The FFN's down projection (rows of F up to 32768; shorter rows skip
    // the segments past their end): one instantiation.
    if (glu) return launch_roll_fused<8, true>(d, count, s);
    if (kmax <= 4096) return launch_roll_fused<1, false>(d, count, s);
    if (kmax <= 8192) return launch_roll_fused<2, false>(d, count, s);
    if (kmax <= 16384) return launch_roll_fused<4, false>(d, count, s);
    return launch_roll_fused<8, false>(d, count, s);
}

}  // namespace bl
