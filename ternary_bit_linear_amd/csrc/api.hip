// api.hip -- the exported C ABI (declared in include/bitlinear.h): host-side
// argument validation, workspace carving and route dispatch.  Every check
// runs before anything is enqueued; no exception leaves this file.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/bitlinear.h"
#include "common.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Row length limit: keeps every per-tile buffer view below 2^31 bytes.
constexpr int64_t kMaxK = int64_t(1) << 22;
// AUTO: decode route up to 4 tokens; from 5 on the MFMA tile kernel, which
// reads the weights once per 32- or 64-token tile, is faster on MI355X
// (measured at K = N = 8192 and on the 70B FFN shapes, M = 4, 8, 16).
// 2..4 tokens whose block the one-shot and rolling decode forms do not hold
// (M * K past 64 KB) take the tile kernel too: the decode route would take
// its persistent form there (70B down projection, K = 28672, at M = 4:
// 28.2 against 23.1 us per forward).
constexpr int kGemvMaxM = 4;
using bl::kFuseMaxLds;
using bl::kFuseMaxM;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

bl_status check_mk(int64_t M, int64_t K) {
    if (M < 1 || K < 1 || K % bl::kBlockWeights != 0 || K > kMaxK) return BL_ERR_SHAPE;
    if (M > kMaxDim || K > kMaxDim || M * K >= kMaxElems) return BL_ERR_SHAPE;
    return BL_OK;
}

bl_status check_nk(int64_t N, int64_t K) {
    if (N < 1 || K < 1 || K % bl::kBlockWeights != 0 || K > kMaxK) return BL_ERR_SHAPE;
    if (N > kMaxDim || K > kMaxDim || N * K >= kMaxElems) return BL_ERR_SHAPE;
    // grids of the pack kernels: N*K/16 words in 256-thread blocks
    if ((N * (K / 16) + 255) / 256 > kMaxDim) return BL_ERR_SHAPE;
    return BL_OK;
}

bl_status check_mn(int64_t M, int64_t N) {
    if (M * N >= kMaxElems) return BL_ERR_SHAPE;
    return BL_OK;
}

bl_status check_launch(const bl_launch *l, bool forward) {
    if (!l) return BL_OK;
    if (l->path < BL_PATH_AUTO || l->path > BL_PATH_GEMM) return BL_ERR_INVALID_ARG;
    if (l->fuse < -1 || l->fuse > 1 || (!forward && l->fuse == 1)) return BL_ERR_INVALID_ARG;
    if (l->reserved != 0) return BL_ERR_INVALID_ARG;
    if (l->variant < 0) return BL_ERR_INVALID_ARG;
    if (l->variant > 0) {
        const int path = l->path == BL_PATH_AUTO ? 0 : l->path;
        if (path == 0) return BL_ERR_INVALID_ARG;  // a variant needs an explicit route
        const int nv = path == BL_PATH_GEMV ? bl::gemv_num_variants() : bl::gemm_num_variants();
        if (l->variant > nv) return BL_ERR_INVALID_ARG;
    }
    return BL_OK;
}

inline bl_status hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

struct Workspace {
    int8_t *q;
    float *inv;
    int32_t *qsum;
};

Workspace carve(void *ws, int64_t M, int64_t K) {
    uint8_t *p = static_cast<uint8_t *>(ws);
    Workspace w;
    w.q = reinterpret_cast<int8_t *>(p);
    p += align256((size_t)(M * K));
    w.inv = reinterpret_cast<float *>(p);
    p += align256((size_t)M * 4);
    w.qsum = reinterpret_cast<int32_t *>(p);
    return w;
}

// The contraction route a launch takes for M tokens of rows of K.
int route_of(int64_t M, int64_t K, const bl_launch *l) {
    const int path = l ? l->path : BL_PATH_AUTO;
    if (path != BL_PATH_AUTO) return path;
    if (M == 1) return BL_PATH_GEMV;
    return M <= kGemvMaxM && bl::roll_supported(M, K) ? BL_PATH_GEMV : BL_PATH_GEMM;
}

// Launch-grid row limit of a route: 16 tokens per decode workgroup row,
// 32 per row of the smallest prefill tile, at most 65535 rows (either route
// fits the few tokens whose automatic route depends on K).
bl_status check_grid(int64_t M, const bl_launch *l) {
    const int path = l ? l->path : BL_PATH_AUTO;
    const bool gemv = path == BL_PATH_GEMV || (path == BL_PATH_AUTO && M <= kGemvMaxM);
    const int64_t rows = gemv ? (M + 15) / 16 : (M + 31) / 32;
    return rows > 65535 ? BL_ERR_SHAPE : BL_OK;
}

// Contraction with q / inv / qsum already computed: route choice and
// launch, with y (rescale epilogue) or acc (int32 epilogue).
bl_status run_contraction(const int8_t *q, const float *inv, const int32_t *qsum,
                          const uint8_t *packed, float w_scale, int64_t M, int64_t K,
                          int64_t N, float *y, int32_t *acc, const bl_launch *l, hipStream_t s) {
    if (bl_status st = check_grid(M, l)) return st;
    const int variant = l ? l->variant : 0;
    if (route_of(M, K, l) == BL_PATH_GEMV)
        return hip_status(bl::launch_gemv(q, inv, qsum, packed, w_scale, M, K, N, y, acc,
                                          variant, s));
    return hip_status(bl::launch_gemm(q, inv, qsum, packed, w_scale, M, K, N, y, acc, variant, s));
}

bl_status validate_forward(const bl_forward_desc &d, const bl_launch *launch) {
    if (bl_status st = check_mk(d.M, d.K)) return st;
    if (bl_status st = check_nk(d.N, d.K)) return st;
    if (bl_status st = check_mn(d.M, d.N)) return st;
    // gamma == nullptr: no RMSNorm, and eps is not used.
    if (!d.x || !d.packed_w || !d.y || !d.workspace) return BL_ERR_INVALID_ARG;
    if ((d.gamma && (!(d.eps > 0.0f) || !std::isfinite(d.eps))) || !std::isfinite(d.w_scale))
        return BL_ERR_INVALID_ARG;
    if (bl_status st = check_launch(launch, true)) return st;
    if (!aligned16(d.x) || !aligned16(d.gamma) || !aligned16(d.packed_w) || !aligned16(d.y) ||
        !aligned16(d.workspace))
        return BL_ERR_ALIGN;
    if (d.workspace_bytes < bitlinear_workspace_bytes(d.M, d.K)) return BL_ERR_WORKSPACE;
    const bool gemv = route_of(d.M, d.K, launch) == BL_PATH_GEMV;
    const bool fits = d.M <= kFuseMaxM && d.M * d.K <= kFuseMaxLds;
    if (launch && launch->fuse == 1 && !(gemv && fits)) return BL_ERR_INVALID_ARG;
    return check_grid(d.M, launch);
}

constexpr int kFusedPerLaunch = 8;

bl::FusedDecode fused_of(const bl_forward_desc &d) {
    const Workspace ws = carve(d.workspace, d.M, d.K);
    bl::FusedDecode f;
    f.x = d.x;
    f.gamma = d.gamma;
    f.packed = d.packed_w;
    f.y = d.y;
    f.q = ws.q;
    f.inv = ws.inv;
    f.qsum = ws.qsum;
    f.eps = d.eps;
    f.w_scale = d.w_scale;
    f.M = d.M;
    f.K = d.K;
    f.N = d.N;
    return f;
}

// Whether a validated forward takes the fused decode kernel.  Automatic
// choice: fused for one token (rows up to 32768: the one-shot kernel holds
// rows up to 8192 in the registers of its 256-thread quantisation, the
// rolling kernel rows up to 32768 in those of its 1024 threads), and for 2
// or 3 tokens with rows up to 8192 (their sets go out fused when the
// one-shot kernel's 16-wave shape holds them in one round, else as the
// separate quantisation + contraction pair; measured on MI355X).
bool takes_fused(const bl_forward_desc &d, const bl_launch *launch) {
    const bool gemv = route_of(d.M, d.K, launch) == BL_PATH_GEMV;
    const bool fits = d.M <= kFuseMaxM && d.M * d.K <= kFuseMaxLds;
    if (launch && launch->fuse == 0) return false;
    if (launch && launch->fuse == 1) return gemv && fits;
    if (d.M == 1) return gemv && fits && (d.K <= 8 * 1024 || bl::roll_fused_supported(d.M, d.K));
    return gemv && fits && d.M <= bl::kFewFusedMaxM && d.K <= 8 * 1024 &&
           bl::shot_fused_supported(d.M, d.K);
}


// Whether a validated forward that does not take the fused kernel can join
// a grouped prefill launch (one batched quantisation launch, one grouped
// tile-kernel launch): automatic launch shape, the tile route, K a whole
// number of 256-k steps and rows that the batched quantisation holds in
// registers.
bool takes_group(const bl_forward_desc &d, const bl_launch *launch) {
    if (launch && launch->variant != 0) return false;
    return route_of(d.M, d.K, launch) == BL_PATH_GEMM && bl::gemm_group_supported(d.K) &&
           d.K <= bl::kActQuantBatchMaxK;
}

// Whether a validated forward that does not take the fused kernel joins a
// batched decode launch pair (one batched quantisation launch, one one-shot
// contraction launch over up to 8 problems): automatic launch shape, not
// forced onto the tile route, and a token block the one-shot kernel holds
// (M <= 8, M * K <= 64 KB, K <= 8192).  Measured on MI355X against two
// launches per BitLinear at M = 2..4 (decoder layer at M = 4: 47 -> 12 us)
// and against the grouped tile pair at M = 5..8 (decoder layer at M = 8:
// 14.7 -> 13.8 us; K = N = 8192: 13.6 -> 11.6 us).
bool takes_shot_batch(const bl_forward_desc &d, const bl_launch *launch) {
    if (launch && (launch->variant != 0 || launch->path == BL_PATH_GEMM)) return false;
    return bl::shot_supported(d.M, d.K) && d.K <= bl::kActQuantBatchMaxK;
}

// Enqueue one validated forward that does not take the fused kernel.
bl_status enqueue_unfused(const bl_forward_desc &d, const bl_launch *launch, hipStream_t s) {
    const Workspace ws = carve(d.workspace, d.M, d.K);
    if (bl::launch_act_quant(d.x, d.gamma, d.eps, d.M, d.K, ws.q, ws.inv, ws.qsum, s) !=
        hipSuccess)
        return BL_ERR_HIP;
    return run_contraction(ws.q, ws.inv, ws.qsum, d.packed_w, d.w_scale, d.M, d.K, d.N, d.y,
                           nullptr, launch, s);
}

// FFN block workspace: g, u (fp32 [M][F] each), then the gate, up and down
// projections' own forward workspaces.
struct FfnWorkspace {
    float *g, *u;
    void *ws_gate, *ws_up, *ws_down;
    size_t b_gate, b_down;
    float *a;  // relu2_mul(g, u), only when F > kActQuantBatchMaxK
};

FfnWorkspace carve_ffn(void *ws, int64_t M, int64_t H, int64_t F) {
    uint8_t *p = static_cast<uint8_t *>(ws);
    FfnWorkspace w;
    const size_t gb = align256((size_t)(M * F) * 4);
    w.g = reinterpret_cast<float *>(p);
    w.u = reinterpret_cast<float *>(p + gb);
    p += 2 * gb;
    w.b_gate = align256(bitlinear_workspace_bytes(M, H));
    w.b_down = align256(bitlinear_workspace_bytes(M, F));
    w.ws_gate = p;
    w.ws_up = p + w.b_gate;
    w.ws_down = p + 2 * w.b_gate;
    w.a = reinterpret_cast<float *>(p + 2 * w.b_gate + w.b_down);
    return w;
}

constexpr int kMaxBatchDescs = 64;
constexpr int kGroupPerLaunch = 8;
constexpr int kShotPerLaunch = 8;

bl_status validate_io(const bl_forward_io_desc &d) {
    const int64_t M = d.M, K = d.K, N = d.N;
    if (bl_status st = check_mk(M, K)) return st;
    if (bl_status st = check_nk(N, K)) return st;
    if (bl_status st = check_mn(M, N)) return st;
    if (!d.x || !d.packed_w || !d.y || !d.workspace) return BL_ERR_INVALID_ARG;
    auto known = [](int t) { return t == BL_F32 || t == BL_BF16 || t == BL_F16; };
    if (!known(d.x_dtype) || !known(d.y_dtype)) return BL_ERR_INVALID_ARG;
    if ((d.gamma && (!(d.eps > 0.0f) || !std::isfinite(d.eps))) || !std::isfinite(d.w_scale))
        return BL_ERR_INVALID_ARG;
    if (!aligned16(d.x) || !aligned16(d.gamma) || !aligned16(d.packed_w) || !aligned16(d.y) ||
        !aligned16(d.workspace))
        return BL_ERR_ALIGN;
    if (d.workspace_bytes < bitlinear_io_workspace_bytes(M, K, N)) return BL_ERR_WORKSPACE;
    return check_grid(M, nullptr);
}

// Whether a validated typed forward joins a one-shot fused launch.
bool io_fusable(const bl_forward_io_desc &d) {
    return d.M == 1 && d.K <= 8 * 1024 && d.x_dtype == d.y_dtype &&
           bl::shot_fused_supported(d.M, d.K);
}

bl::FusedDecode fused_io_of(const bl_forward_io_desc &d) {
    const Workspace ws = carve(d.workspace, d.M, d.K);
    bl::FusedDecode f;
    f.x = static_cast<const float *>(d.x);  // of type io, as the kernel reads it
    f.gamma = d.gamma;
    f.packed = d.packed_w;
    f.y = static_cast<float *>(d.y);
    f.q = ws.q;
    f.inv = ws.inv;
    f.qsum = ws.qsum;
    f.eps = d.eps;
    f.w_scale = d.w_scale;
    f.M = d.M;
    f.K = d.K;
    f.N = d.N;
    f.io = d.x_dtype;
    return f;
}

// The three-launch form: typed quantisation, contraction to the int32
// accumulator, typed rescale.
bl_status enqueue_io_staged(const bl_forward_io_desc &d, hipStream_t s) {
    const Workspace ws = carve(d.workspace, d.M, d.K);
    int32_t *acc = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(d.workspace) +
                                               align256(bitlinear_workspace_bytes(d.M, d.K)));
    if (bl::launch_act_quant_io(d.x, d.x_dtype, d.gamma, d.eps, d.M, d.K, ws.q, ws.inv, ws.qsum,
                                s) != hipSuccess)
        return BL_ERR_HIP;
    if (bl_status st = run_contraction(ws.q, ws.inv, ws.qsum, d.packed_w, d.w_scale, d.M, d.K,
                                       d.N, nullptr, acc, nullptr, s))
        return st;
    return hip_status(bl::launch_rescale_io(acc, ws.inv, d.w_scale, d.M, d.N, d.y, d.y_dtype, s));
}

// Fused launches of up to 8 same-type problems when their workgroups fit on
// the device at once; else each one staged.
bl_status flush_io_group(const bl_forward_io_desc *const *g, int n, hipStream_t s) {
    if (n == 0) return BL_OK;
    int64_t Ms[8], Ks[8], Ns[8];
    bl::FusedDecode f[8];
    for (int i = 0; i < n; ++i) {
        Ms[i] = g[i]->M;
        Ks[i] = g[i]->K;
        Ns[i] = g[i]->N;
        f[i] = fused_io_of(*g[i]);
    }
    if (bl::shot_rounds(Ms, Ks, Ns, n, true) == 1)
        return hip_status(bl::launch_gemv_shot_fused(f, n, 0, s));
    for (int i = 0; i < n; ++i)
        if (bl_status st = enqueue_io_staged(*g[i], s)) return st;
    return BL_OK;
}

// Scratch array of the allocation-free forward: one per device (each GPU
// that loads the library's code holds its own copy), held until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host the
// name is only a stand-in); it uses the device address looked up once per
// device with hipGetSymbolAddress.
constexpr size_t kScratchBytes = BITLINEAR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array (looked up on the
// first call on that device, with that device current).
bl_status scratch_of_current_device(void **out);

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

bl_status scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BL_ERR_HIP;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BL_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BL_OK;
}

}  // namespace

extern "C" {

const char *bitlinear_status_string(int status) {
    switch (status) {
        case BL_OK: return "BL_OK";
        case BL_ERR_INVALID_ARG: return "BL_ERR_INVALID_ARG: invalid argument";
        case BL_ERR_SHAPE: return "BL_ERR_SHAPE: size < 1, K % 128 != 0, or too large";
        case BL_ERR_ALIGN: return "BL_ERR_ALIGN: pointer not 16-byte aligned";
        case BL_ERR_NOT_TERNARY: return "BL_ERR_NOT_TERNARY: weights are not ternary x one scale";
        case BL_ERR_WORKSPACE: return "BL_ERR_WORKSPACE: workspace too small";
        case BL_ERR_HIP: return "BL_ERR_HIP: HIP runtime or launch failure";
        default: return "unknown bitlinear status";
    }
}

int bitlinear_abi_version(void) { return 1; }

int bitlinear_num_variants(int path) {
    if (path == BL_PATH_GEMV) return bl::gemv_num_variants();
    if (path == BL_PATH_GEMM) return bl::gemm_num_variants();
    return 0;
}

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
    if (check_nk(N, K) != BL_OK) return 0;
    return (size_t)(N * (K / 4)) + bl::kTrailerBytes;
}

size_t bitlinear_workspace_bytes(int64_t M, int64_t K) {
    if (M < 1 || K < 1 || M > kMaxDim || K > kMaxDim || M * K >= kMaxElems) return 0;
    return align256((size_t)(M * K)) + align256((size_t)M * 4) + align256((size_t)M * 4);
}

bl_status bitlinear_pack_i2s(const float *w, int64_t N, int64_t K, uint8_t *packed,
                             float *w_scale_out, void *stream) {
    if (bl_status st = check_nk(N, K)) return st;
    if (!w || !packed) return BL_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(packed)) return BL_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    uint8_t *trailer = packed + N * (K / 4);
    if (bl::launch_pack_init(trailer, s) != hipSuccess) return BL_ERR_HIP;
    if (bl::launch_pack_scan(w, N, K, packed, s) != hipSuccess) return BL_ERR_HIP;
    uint32_t stats[2] = {0u, 0u};
    if (hipMemcpyAsync(stats, trailer, sizeof stats, hipMemcpyDeviceToHost, s) != hipSuccess)
        return BL_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return BL_ERR_HIP;
    const uint32_t mn = stats[0], mx = stats[1];
    bl_status st = BL_OK;
    float scale = 0.0f;
    if (mx == 0u) {
        scale = 0.0f;  // W == 0: every code 1
    } else if (mn != mx || mx >= 0x7f800000u) {
        st = BL_ERR_NOT_TERNARY;  // two magnitudes, or inf / NaN
    } else {
        std::memcpy(&scale, &mx, sizeof scale);
    }
    if (bl::launch_pack_finalize(trailer, scale, s) != hipSuccess) return BL_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return BL_ERR_HIP;
    if (st == BL_OK && w_scale_out) *w_scale_out = scale;
    return st;
}

bl_status bitlinear_unpack_i2s(const uint8_t *packed, int64_t N, int64_t K, float *w_out,
                               void *stream) {
    if (bl_status st = check_nk(N, K)) return st;
    if (!packed || !w_out) return BL_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(w_out)) return BL_ERR_ALIGN;
    return hip_status(bl::launch_unpack(packed, N, K, w_out, as_stream(stream)));
}

bl_status bitlinear_dequant_i2s(const uint8_t *packed, int64_t N, int64_t K, void *w_out,
                                int w_dtype, void *stream) {
    if (bl_status st = check_nk(N, K)) return st;
    if (!packed || !w_out) return BL_ERR_INVALID_ARG;
    if (w_dtype != BL_F32 && w_dtype != BL_BF16 && w_dtype != BL_F16) return BL_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(w_out)) return BL_ERR_ALIGN;
    return hip_status(bl::launch_dequant(packed, N, K, w_out, w_dtype, as_stream(stream)));
}

bl_status bitlinear_read_scale(const uint8_t *packed, int64_t N, int64_t K, float *out_host,
                               void *stream) {
    if (bl_status st = check_nk(N, K)) return st;
    if (!packed || !out_host) return BL_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    float v = 0.0f;
    if (hipMemcpyAsync(&v, packed + N * (K / 4), sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess)
        return BL_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return BL_ERR_HIP;
    *out_host = v;
    return BL_OK;
}

bl_status bitlinear_act_quant(const float *x, const float *gamma, float eps, int64_t M,
                              int64_t K, int8_t *q, float *inv, int32_t *qsum, void *stream) {
    if (bl_status st = check_mk(M, K)) return st;
    if (!x || !q || !inv || !qsum) return BL_ERR_INVALID_ARG;
    if (gamma && (!(eps > 0.0f) || !std::isfinite(eps))) return BL_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(q)) return BL_ERR_ALIGN;
    return hip_status(bl::launch_act_quant(x, gamma, eps, M, K, q, inv, qsum, as_stream(stream)));
}

bl_status bitlinear_fp32_ops(int op, const float *a, const float *b, float eps, int64_t n,
                             float *out, void *stream) {
    if (n < 1 || n >= kMaxElems) return BL_ERR_SHAPE;
    if (op < BL_FP_SQRT || op > BL_FP_QUANT_SCALE || !a || !out) return BL_ERR_INVALID_ARG;
    if ((op == BL_FP_DIV || op == BL_FP_RMS_SCALE) && !b) return BL_ERR_INVALID_ARG;
    if (op == BL_FP_RMS_SCALE && !std::isfinite(eps)) return BL_ERR_INVALID_ARG;
    return hip_status(bl::launch_fp32_ops(op, a, b, eps, n, out, as_stream(stream)));
}

bl_status bitlinear_matmul_i2s_ex(const int8_t *q, const int32_t *qsum, const uint8_t *packed_w,
                                  int64_t M, int64_t K, int64_t N, int32_t *acc,
                                  const bl_launch *launch, void *stream) {
    if (bl_status st = check_mk(M, K)) return st;
    if (bl_status st = check_nk(N, K)) return st;
    if (bl_status st = check_mn(M, N)) return st;
    if (!q || !qsum || !packed_w || !acc) return BL_ERR_INVALID_ARG;
    if (bl_status st = check_launch(launch, false)) return st;
    if (!aligned16(q) || !aligned16(packed_w)) return BL_ERR_ALIGN;
    return run_contraction(q, nullptr, qsum, packed_w, 0.0f, M, K, N, nullptr, acc, launch,
                           as_stream(stream));
}

bl_status bitlinear_matmul_i2s(const int8_t *q, const int32_t *qsum, const uint8_t *packed_w,
                               int64_t M, int64_t K, int64_t N, int32_t *acc, void *stream) {
    return bitlinear_matmul_i2s_ex(q, qsum, packed_w, M, K, N, acc, nullptr, stream);
}

bl_status bitlinear_forward_ex(const float *x, const uint8_t *packed_w, float w_scale,
                               const float *gamma, float eps, int64_t M, int64_t K, int64_t N,
                               float *y, void *workspace, size_t workspace_bytes,
                               const bl_launch *launch, void *stream) {
    const bl_forward_desc d{x, packed_w, w_scale, gamma, eps, M, K, N, y, workspace,
                            workspace_bytes};
    if (bl_status st = validate_forward(d, launch)) return st;
    hipStream_t s = as_stream(stream);
    if (takes_fused(d, launch)) {
        const bl::FusedDecode f = fused_of(d);
        return hip_status(bl::launch_gemv_fused(&f, 1, launch ? launch->variant : 0, s));
    }
    if (takes_shot_batch(d, launch) || takes_group(d, launch))
        return bitlinear_forward_batch(&d, 1, launch, stream);
    return enqueue_unfused(d, launch, s);
}

bl_status bitlinear_forward(const float *x, const uint8_t *packed_w, float w_scale,
                            const float *gamma, float eps, int64_t M, int64_t K, int64_t N,
                            float *y, void *workspace, size_t workspace_bytes, void *stream) {
    return bitlinear_forward_ex(x, packed_w, w_scale, gamma, eps, M, K, N, y, workspace,
                                workspace_bytes, nullptr, stream);
}

size_t bitlinear_probe_read_sink_words(size_t bytes) {
    if (bytes < 16 || bytes % 16 != 0 || bytes >= ((size_t)1 << 40)) return 0;
    return (size_t)bl::probe_read_blocks(bytes);
}

bl_status bitlinear_probe_read(const void *src, size_t bytes, uint32_t *sink, size_t sink_words,
                               void *stream) {
    const size_t need = bitlinear_probe_read_sink_words(bytes);
    if (need == 0 || need > (size_t)kMaxDim) return BL_ERR_SHAPE;
    if (!src || !sink || sink_words < need) return BL_ERR_INVALID_ARG;
    if (!aligned16(src)) return BL_ERR_ALIGN;
    return hip_status(bl::launch_probe_read(static_cast<const uint8_t *>(src), bytes, sink,
                                            as_stream(stream)));
}

bl_status bitlinear_probe_mfma(int64_t iters, int64_t workgroups, int32_t *sink,
                               size_t sink_words, void *stream) {
    if (iters < 1 || workgroups < 1 || workgroups > kMaxDim) return BL_ERR_SHAPE;
    if (!sink || sink_words < (size_t)workgroups * 256) return BL_ERR_INVALID_ARG;
    return hip_status(bl::launch_probe_mfma(iters, workgroups, sink, as_stream(stream)));
}

bl_status bitlinear_forward_noalloc(const float *x, const uint8_t *packed_w, float w_scale,
                                    const float *gamma, float eps, int64_t M, int64_t K, int64_t N,
                                    float *y, void *stream) {
    // Every host-side check first (the aligned stand-in address is never
    // dereferenced), then the size limit, then the scratch address.
    const bl_forward_desc probe{x, packed_w, w_scale, gamma, eps, M, K, N, y,
                                reinterpret_cast<void *>(uintptr_t(256)), kScratchBytes};
    if (bl_status st = validate_forward(probe, nullptr)) return st;
    void *ws = nullptr;
    if (bl_status st = scratch_of_current_device(&ws)) return st;
    return bitlinear_forward_ex(x, packed_w, w_scale, gamma, eps, M, K, N, y, ws, kScratchBytes,
                                nullptr, stream);
}

size_t bitlinear_io_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (check_mk(M, K) || N < 1 || N > kMaxDim || check_mn(M, N)) return 0;
    return align256(bitlinear_workspace_bytes(M, K)) + align256((size_t)(M * N) * 4);
}

bl_status bitlinear_forward_io_batch(const bl_forward_io_desc *descs, int count, void *stream) {
    if (!descs || count < 1 || count > kMaxBatchDescs) return BL_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i)
        if (bl_status st = validate_io(descs[i])) return st;
    hipStream_t s = as_stream(stream);
    const bl_forward_io_desc *grp[3][8];
    int n[3] = {0, 0, 0};
    // Prefill-sized problems: one batched typed quantisation and one grouped
    // tile launch (typed epilogue) per 8 of one (x type, y type) pair.
    struct PrefillGroup {
        bl::ActQuantDesc aq[kGroupPerLaunch];
        bl::GemmDesc gd[kGroupPerLaunch];
        int n = 0;
    };
    PrefillGroup pg[3][3];
    auto flush_pg = [&](PrefillGroup &G) -> bl_status {
        if (G.n == 0) return BL_OK;
        if (bl::launch_act_quant_batch(G.aq, G.n, s) != hipSuccess) return BL_ERR_HIP;
        if (bl::launch_gemm_group(G.gd, G.n, s) != hipSuccess) return BL_ERR_HIP;
        G.n = 0;
        return BL_OK;
    };
    // A few tokens (M <= 8, M * K <= 64 KB), and one token with x and y of
    // different types: one batched typed quantisation and one one-shot
    // contraction launch (typed epilogue) per 8 of one type pair.
    struct ShotGroup {
        bl::ActQuantDesc aq[kShotPerLaunch];
        bl::ShotDecode sd[kShotPerLaunch];
        int n = 0;
    };
    ShotGroup sgp[3][3];
    auto flush_sg = [&](ShotGroup &G) -> bl_status {
        if (G.n == 0) return BL_OK;
        if (bl::launch_act_quant_batch(G.aq, G.n, s) != hipSuccess) return BL_ERR_HIP;
        if (bl::launch_gemv_shot(G.sd, G.n, 0, s) != hipSuccess) return BL_ERR_HIP;
        G.n = 0;
        return BL_OK;
    };
    for (int i = 0; i < count; ++i) {
        const bl_forward_io_desc &d = descs[i];
        if (!io_fusable(d)) {
            if (bl::shot_supported(d.M, d.K) && d.K <= bl::kActQuantBatchMaxK) {
                ShotGroup &G = sgp[d.x_dtype][d.y_dtype];
                const Workspace ws = carve(d.workspace, d.M, d.K);
                bl::ActQuantDesc &a = G.aq[G.n];
                a = bl::ActQuantDesc{d.x, d.gamma, d.eps, d.M, d.K, ws.q, ws.inv, ws.qsum};
                a.io = d.x_dtype;
                bl::ShotDecode &c = G.sd[G.n];
                c = bl::ShotDecode{ws.q,    ws.inv,    ws.qsum, d.packed_w, static_cast<float *>(d.y),
                                   nullptr, d.w_scale, d.M,     d.K,        d.N};
                c.io = d.y_dtype;
                if (++G.n == kShotPerLaunch)
                    if (bl_status st = flush_sg(G)) return st;
                continue;
            }
            if (route_of(d.M, d.K, nullptr) == BL_PATH_GEMM && bl::gemm_group_supported(d.K) &&
                d.K <= bl::kActQuantBatchMaxK) {
                PrefillGroup &G = pg[d.x_dtype][d.y_dtype];
                const Workspace ws = carve(d.workspace, d.M, d.K);
                bl::ActQuantDesc &a = G.aq[G.n];
                a = bl::ActQuantDesc{d.x, d.gamma, d.eps, d.M, d.K, ws.q, ws.inv, ws.qsum};
                a.io = d.x_dtype;
                bl::GemmDesc &g = G.gd[G.n];
                g = bl::GemmDesc{ws.q, ws.inv, ws.qsum, d.packed_w, d.w_scale, d.M, d.K, d.N,
                                 static_cast<float *>(d.y), nullptr};
                g.io = d.y_dtype;
                if (++G.n == kGroupPerLaunch)
                    if (bl_status st = flush_pg(G)) return st;
            } else if (bl_status st = enqueue_io_staged(d, s)) {
                return st;
            }
            continue;
        }
        const int t = d.x_dtype;
        grp[t][n[t]++] = &d;
        if (n[t] == 8) {
            if (bl_status st = flush_io_group(grp[t], 8, s)) return st;
            n[t] = 0;
        }
    }
    for (int t = 0; t < 3; ++t)
        if (bl_status st = flush_io_group(grp[t], n[t], s)) return st;
    for (int xt = 0; xt < 3; ++xt)
        for (int yt = 0; yt < 3; ++yt) {
            if (bl_status st = flush_sg(sgp[xt][yt])) return st;
            if (bl_status st = flush_pg(pg[xt][yt])) return st;
        }
    return BL_OK;
}

bl_status bitlinear_forward_io(const void *x, int x_dtype, const uint8_t *packed_w, float w_scale,
                               const float *gamma, float eps, int64_t M, int64_t K, int64_t N,
                               void *y, int y_dtype, void *workspace, size_t workspace_bytes,
                               void *stream) {
    const bl_forward_io_desc d{x,   x_dtype, packed_w, w_scale, gamma,          eps,
                               M,   K,       N,        y,       y_dtype,        workspace,
                               workspace_bytes};
    return bitlinear_forward_io_batch(&d, 1, stream);
}

size_t bitlinear_ffn_workspace_bytes(int64_t M, int64_t H, int64_t F) {
    if (check_mk(M, H) || check_mk(M, F) || check_mn(M, F) || check_mn(M, H)) return 0;
    const size_t gb = align256((size_t)(M * F) * 4);
    return 2 * gb + 2 * align256(bitlinear_workspace_bytes(M, H)) +
           align256(bitlinear_workspace_bytes(M, F)) + (F > bl::kActQuantBatchMaxK ? gb : 0);
}

bl_status bitlinear_ffn_forward(const bl_ffn_desc *desc, void *stream) {
    if (!desc) return BL_ERR_INVALID_ARG;
    const bl_ffn_desc &d = *desc;
    const int64_t M = d.M, H = d.H, F = d.F;
    if (bl_status st = check_mk(M, H)) return st;
    if (bl_status st = check_mk(M, F)) return st;
    if (bl_status st = check_nk(F, H)) return st;
    if (bl_status st = check_nk(H, F)) return st;
    if (bl_status st = check_mn(M, F)) return st;
    if (bl_status st = check_mn(M, H)) return st;
    if (!d.x || !d.packed_gate || !d.packed_up || !d.packed_down || !d.y || !d.workspace)
        return BL_ERR_INVALID_ARG;
    if ((d.gamma_in || d.gamma_sub) && (!(d.eps > 0.0f) || !std::isfinite(d.eps)))
        return BL_ERR_INVALID_ARG;
    if (!std::isfinite(d.s_gate) || !std::isfinite(d.s_up) || !std::isfinite(d.s_down))
        return BL_ERR_INVALID_ARG;
    if (!aligned16(d.x) || !aligned16(d.gamma_in) || !aligned16(d.gamma_sub) ||
        !aligned16(d.packed_gate) || !aligned16(d.packed_up) || !aligned16(d.packed_down) ||
        !aligned16(d.y) || !aligned16(d.workspace))
        return BL_ERR_ALIGN;
    if (d.workspace_bytes < bitlinear_ffn_workspace_bytes(M, H, F)) return BL_ERR_WORKSPACE;
    if (bl_status st = check_grid(M, nullptr)) return st;
    const FfnWorkspace w = carve_ffn(d.workspace, M, H, F);
    // 1. gate and up: two BitLinears over the same x.
    hipStream_t s = as_stream(stream);
    const bl_forward_desc gu[2] = {
        {d.x, d.packed_gate, d.s_gate, d.gamma_in, d.eps, M, H, F, w.g, w.ws_gate, w.b_gate},
        {d.x, d.packed_up, d.s_up, d.gamma_in, d.eps, M, H, F, w.u, w.ws_up, w.b_gate}};
    // (A few tokens take the fused kernel only where its 16-wave shape
    // holds gate and up in one round; else x is quantised once below.)
    const int64_t gM[2] = {M, M}, gK[2] = {H, H}, gN[2] = {F, F};
    const bool fuse_gu = takes_fused(gu[0], nullptr) &&
                         (M == 1 || bl::few_fused_one_round(gM, gK, gN, 2));
    if (!fuse_gu && takes_shot_batch(gu[0], nullptr)) {
        // A few tokens: x is quantised once (into the gate's workspace) and
        // both contractions read that q in one one-shot launch.
        const Workspace wq = carve(w.ws_gate, M, H);
        const bl::ActQuantDesc aq{d.x, d.gamma_in, d.eps, M, H, wq.q, wq.inv, wq.qsum};
        const bl::ShotDecode sd[2] = {
            {wq.q, wq.inv, wq.qsum, d.packed_gate, w.g, nullptr, d.s_gate, M, H, F},
            {wq.q, wq.inv, wq.qsum, d.packed_up, w.u, nullptr, d.s_up, M, H, F}};
        if (bl::launch_act_quant_batch(&aq, 1, s) != hipSuccess ||
            bl::launch_gemv_shot_auto(sd, 2, s) != hipSuccess)
            return BL_ERR_HIP;
    } else if (!fuse_gu && takes_group(gu[0], nullptr)) {
        // Prefill: x is quantised once (into the gate's workspace) and both
        // contractions read that q in one grouped tile launch.
        const Workspace wq = carve(w.ws_gate, M, H);
        const bl::ActQuantDesc aq{d.x, d.gamma_in, d.eps, M, H, wq.q, wq.inv, wq.qsum};
        const bl::GemmDesc gd[2] = {
            {wq.q, wq.inv, wq.qsum, d.packed_gate, d.s_gate, M, H, F, w.g, nullptr},
            {wq.q, wq.inv, wq.qsum, d.packed_up, d.s_up, M, H, F, w.u, nullptr}};
        if (bl::launch_act_quant_batch(&aq, 1, s) != hipSuccess ||
            bl::launch_gemm_group(gd, 2, s) != hipSuccess)
            return BL_ERR_HIP;
    } else if (bl_status st = bitlinear_forward_batch(gu, 2, nullptr, stream)) {
        return st;
    }
    // 2. down over relu2_mul(g, u), formed while its quantisation reads g, u.
    const Workspace wd = carve(w.ws_down, M, F);
    const int64_t Ms[1] = {M}, Ks[1] = {F}, Ns[1] = {H};
    const bool shot_glu = M == 1 && F <= 8 * 1024 && bl::shot_fused_supported(M, F) &&
                          bl::shot_rounds(Ms, Ks, Ns, 1, true, true) == 1;
    if (shot_glu || (M == 1 && bl::roll_fused_supported(M, F))) {
        // One launch: the down projection's quantisation forms relu2(g) * u
        // as it reads g and u (the one-shot kernel when its workgroups fit
        // the device at once, else the rolling kernel).
        bl::FusedDecode f;
        f.x = w.g;
        f.gamma = d.gamma_sub;
        f.packed = d.packed_down;
        f.y = d.y;
        f.q = wd.q;
        f.inv = wd.inv;
        f.qsum = wd.qsum;
        f.eps = d.eps;
        f.w_scale = d.s_down;
        f.M = M;
        f.K = F;
        f.N = H;
        f.u = w.u;
        return hip_status(shot_glu ? bl::launch_gemv_shot_fused(&f, 1, 0, s)
                                   : bl::launch_gemv_roll_fused(&f, 1, s));
    }
    if (F <= bl::kActQuantBatchMaxK) {
        // rows in registers: the product is formed inside the quantisation
        if (bl::launch_act_quant_glu(w.g, w.u, d.gamma_sub, d.eps, M, F, wd.q, wd.inv, wd.qsum,
                                     s) != hipSuccess)
            return BL_ERR_HIP;
    } else {
        // longer rows: one elementwise pass, then the quantisation that
        // holds rows up to 32768 in registers (measured faster than a
        // streamed gated quantisation at F = 28672)
        if (bl::launch_relu2_mul(w.g, w.u, w.a, M * F, s) != hipSuccess ||
            bl::launch_act_quant(w.a, d.gamma_sub, d.eps, M, F, wd.q, wd.inv, wd.qsum, s) !=
                hipSuccess)
            return BL_ERR_HIP;
    }
    if (F <= bl::kActQuantBatchMaxK && bl::shot_supported(M, F)) {
        // the one-shot kernel, as a batch of a few tokens takes it
        const bl::ShotDecode sd{wd.q, wd.inv, wd.qsum, d.packed_down, d.y, nullptr, d.s_down,
                                M,    F,      H};
        return hip_status(bl::launch_gemv_shot_auto(&sd, 1, s));
    }
    return run_contraction(wd.q, wd.inv, wd.qsum, d.packed_down, d.s_down, M, F, H, d.y, nullptr,
                           nullptr, s);
}

bl_status bitlinear_forward_batch(const bl_forward_desc *descs, int count,
                                  const bl_launch *launch, void *stream) {
    if (!descs || count < 1 || count > kMaxBatchDescs) return BL_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i)
        if (bl_status st = validate_forward(descs[i], launch)) return st;
    hipStream_t s = as_stream(stream);
    const int variant = launch ? launch->variant : 0;
    bl::FusedDecode group[kFusedPerLaunch];
    int n = 0;
    bl::ActQuantDesc aq[kGroupPerLaunch];
    bl::GemmDesc gd[kGroupPerLaunch];
    int g = 0;
    auto flush_group = [&]() -> bl_status {
        if (g == 0) return BL_OK;
        if (bl::launch_act_quant_batch(aq, g, s) != hipSuccess) return BL_ERR_HIP;
        if (bl::launch_gemm_group(gd, g, s) != hipSuccess) return BL_ERR_HIP;
        g = 0;
        return BL_OK;
    };
    bl::ActQuantDesc sq[kShotPerLaunch];
    bl::ShotDecode sd[kShotPerLaunch];
    int ns = 0;
    auto flush_shot = [&]() -> bl_status {
        if (ns == 0) return BL_OK;
        if (bl::launch_act_quant_batch(sq, ns, s) != hipSuccess) return BL_ERR_HIP;
        if (bl::launch_gemv_shot_auto(sd, ns, s) != hipSuccess) return BL_ERR_HIP;
        ns = 0;
        return BL_OK;
    };
    auto flush_fused = [&]() -> bl_status {
        if (n > 0 && bl::launch_gemv_fused(group, n, variant, s) != hipSuccess) return BL_ERR_HIP;
        n = 0;
        return BL_OK;
    };
    for (int i = 0; i < count; ++i) {
        const bl_forward_desc &d = descs[i];
        if (takes_fused(d, launch)) {
            group[n++] = fused_of(d);
            if (n == kFusedPerLaunch)
                if (bl_status st = flush_fused()) return st;
        } else if (takes_shot_batch(d, launch)) {
            const Workspace ws = carve(d.workspace, d.M, d.K);
            sq[ns] = bl::ActQuantDesc{d.x, d.gamma, d.eps, d.M, d.K, ws.q, ws.inv, ws.qsum};
            sd[ns] = bl::ShotDecode{ws.q,   ws.inv, ws.qsum, d.packed_w, d.y,
                                    nullptr, d.w_scale, d.M, d.K, d.N};
            if (++ns == kShotPerLaunch)
                if (bl_status st = flush_shot()) return st;
        } else if (takes_group(d, launch)) {
            const Workspace ws = carve(d.workspace, d.M, d.K);
            aq[g] = bl::ActQuantDesc{d.x, d.gamma, d.eps, d.M, d.K, ws.q, ws.inv, ws.qsum};
            gd[g] = bl::GemmDesc{ws.q, ws.inv, ws.qsum, d.packed_w, d.w_scale,
                                 d.M, d.K, d.N, d.y, nullptr};
            if (++g == kGroupPerLaunch)
                if (bl_status st = flush_group()) return st;
        } else if (bl_status st = enqueue_unfused(d, launch, s)) {
            return st;
        }
    }
    if (bl_status st = flush_fused()) return st;
    if (bl_status st = flush_shot()) return st;
    return flush_group();
}

}  // extern "C"
