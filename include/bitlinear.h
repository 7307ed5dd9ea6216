/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) ternary BitLinear library.
 *
 * The library computes the BitNet b1.58 BitLinear forward pass over I2_S
 * packed ternary weights:
 *
 *   RMSNorm of each activation row  ->  per-row absmax int8 quantisation
 *   ->  ternary-code x int8 contraction with int32 accumulation, minus the
 *       activation sum  ->  rescale to fp32.
 *
 * Sources (web pages, cited by title and section):
 *   [HF-38087] huggingface/transformers PR #38087 "Add optional RMSNorm
 *              support to BitNet quantization (config + layers)", section
 *              "What does this PR do?": RMSNorm (eps default 1e-6) is applied
 *              to the activations before quantisation.
 *   [CPPB-7]   eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout +
 *              squared-ReLU FFN": summary bullets "I2_S NEON kernel for the
 *              canonical layout" and "llama-quantize I2_S emits the canonical
 *              layout", section "Known gaps", and the commit messages of the
 *              NEON kernel and of the I2_S quantizer.
 *
 * Conventions shared by every entry point
 *   - W is [N][K] row-major (K contiguous), x is fp32 [M][K] row-major, y is
 *     fp32 [M][N] row-major, gamma is fp32 [K]; y = RMSNorm/quant(x) W^T.
 *   - Every array pointer is a DEVICE pointer owned by the caller, except
 *     where a parameter says "host".  The library allocates no device memory
 *     and keeps no mutable global state, except the per-device scratch array
 *     of bitlinear_forward_noalloc; calls on different streams may run
 *     concurrently (bitlinear_forward_noalloc excepted).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failing check returns its status and enqueues nothing.  No C++
 *     exception crosses this interface and the library never aborts.
 *   - Preconditions checked everywhere they apply: M, N, K >= 1 and
 *     K % 128 == 0 (rows are whole I2_S blocks, [CPPB-7] "Known gaps")
 *     -> BL_ERR_SHAPE; non-NULL pointers -> BL_ERR_INVALID_ARG; x, y, q,
 *     packed_w and the workspace 16-byte aligned -> BL_ERR_ALIGN.
 *   - Sizes are limited to M*K, N*K/4 and M*N below 2^40 elements, to
 *     M, N < 2^31 and to K <= 2^22 (BL_ERR_SHAPE beyond).  Launch grids
 *     add M <= 1048560 on the decode route and M <= 2097120 on the prefill
 *     route (BL_ERR_SHAPE beyond).
 *
 * I2_S packed weight buffer (the persistent format) [CPPB-7]
 *   N*K/4 bytes of 2-bit codes followed by a 32-byte trailer.  Each run of
 *   128 weights of a row (a block) takes 32 bytes: weight j of the block is
 *   in byte j % 32, field j / 32, field g in bits (7-2g)..(6-2g).  The stored
 *   code is w/scale + 1 (-1 -> 0, 0 -> 1, +1 -> 2); consumers subtract the
 *   activation sum.  The trailer is the per-tensor scale (fp32, little
 *   endian) followed by 28 zero bytes.  Row n occupies bytes
 *   [n*K/4, (n+1)*K/4).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BL_OK = 0,
    BL_ERR_INVALID_ARG = 1, /* NULL pointer, bad enum, non-positive eps ...  */
    BL_ERR_SHAPE = 2,       /* size < 1, K % 128 != 0, or too large          */
    BL_ERR_ALIGN = 3,       /* a pointer that must be 16-byte aligned is not */
    BL_ERR_NOT_TERNARY = 4, /* pack: input is not ternary x one scale        */
    BL_ERR_WORKSPACE = 5,   /* workspace smaller than bitlinear_workspace_bytes */
    BL_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed    */
} bl_status;

/* Matmul route.  Both routes return bit-identical results; the choice only
 * affects speed.  AUTO takes the decode kernels for M <= 4 and the MFMA
 * tile kernel above, except that a forward of M <= 8 tokens whose block
 * fits the one-shot decode kernel (M * K <= 65536, K <= 8192) takes that
 * kernel (see bitlinear_forward_batch), and that 2..4 tokens with
 * M * K > 65536 (a block the one-shot and rolling decode forms do not
 * hold) take the tile kernel. */
typedef enum {
    BL_PATH_AUTO = 0,
    BL_PATH_GEMV = 1, /* decode kernel, any M (tokens in groups of 16) */
    BL_PATH_GEMM = 2  /* prefill tile kernel, any M                    */
} bl_path;

/* Launch options for bitlinear_forward_ex / bitlinear_matmul_i2s_ex.
 *   path:    a bl_path value.
 *   fuse:    forward only.  -1 = automatic (fused for M == 1 and
 *            K <= 32768); 0 = separate quantisation kernel; 1 = RMSNorm +
 *            quantisation recomputed inside every workgroup of the decode
 *            kernel (GEMV route only, M <= 4 and M*K <= 32768).
 *   variant: 0 = automatic; otherwise an index into the route's table of
 *            launch shapes (1..bitlinear_num_variants(path)); every variant
 *            returns bit-identical results.
 * Unknown values -> BL_ERR_INVALID_ARG. */
typedef struct {
    int32_t path;
    int32_t fuse;
    int32_t variant;
    int32_t reserved; /* must be 0 */
} bl_launch;

/* Human-readable name of a status value (static string, never NULL). */
const char *bitlinear_status_string(int status);

/* Library ABI version (this header: 1). */
int bitlinear_abi_version(void);

/* Number of launch-shape variants of a route (BL_PATH_GEMV or BL_PATH_GEMM);
 * 0 for anything else. */
int bitlinear_num_variants(int path);

/* Bytes of an I2_S buffer for an N x K tensor: N*K/4 + 32.  Returns 0 when
 * N < 1, K < 1 or K % 128 != 0. */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Bytes of workspace bitlinear_forward needs for M rows of length K: int8
 * q[M][K], fp32 inv[M], int32 qsum[M], each segment 256-byte aligned.
 * Returns 0 when M < 1 or K < 1. */
size_t bitlinear_workspace_bytes(int64_t M, int64_t K);

/* I2_S packer [CPPB-7, summary bullet "llama-quantize I2_S emits the
 * canonical layout", and "Known gaps": scale = first non-zero |w|, input
 * must be ternary x scale, rows divisible by 128].
 *   w:           device, fp32 [N][K]; every value must be 0 or +-s for one
 *                finite s (-0.0 counts as 0).
 *   packed:      device, bitlinear_packed_bytes(N, K) bytes, 16-byte aligned;
 *                written with the codes and the trailer.
 *   w_scale_out: HOST pointer, may be NULL; receives s (0.0f when W == 0).
 * Synchronous: returns after the work on `stream` has finished.  Returns
 * BL_ERR_NOT_TERNARY when two non-zero magnitudes differ or a value is not
 * finite; `packed` is then unspecified (its trailer scale reads 0). */
bl_status bitlinear_pack_i2s(const float *w, int64_t N, int64_t K,
                             uint8_t *packed, float *w_scale_out, void *stream);

/* Unpacker (the to_float direction of the format) [CPPB-7, NEON-kernel
 * commit]: w_out[n][k] = (code(n,k) - 1) * s, s read from the trailer.
 *   packed: device, as written by bitlinear_pack_i2s.
 *   w_out:  device, fp32 [N][K], 16-byte aligned.
 * Asynchronous on `stream`.  A stored code 3 (never written by the packer)
 * decodes to +2*s. */
bl_status bitlinear_unpack_i2s(const uint8_t *packed, int64_t N, int64_t K,
                               float *w_out, void *stream);

/* Reads the per-tensor scale from the trailer into *out_host (HOST pointer).
 * Synchronous on `stream`. */
bl_status bitlinear_read_scale(const uint8_t *packed, int64_t N, int64_t K,
                               float *out_host, void *stream);

/* BitLinear forward [HF-38087 "What does this PR do?" for the RMSNorm before
 * quantisation; CPPB-7 NEON-kernel commit for the i2 x i8 contraction and
 * the activation-sum offset]:
 *   r_m    = 1 / sqrt(sum_k x[m][k]^2 / K + eps)          (fp32)
 *   xn     = (x[m][k] * r_m) * gamma[k]                  (fp32)
 *   inv_m  = 127 / max(max_k |xn|, 1e-5)                 (fp32)
 *   q      = clamp(round_half_even(xn * inv_m), -128, 127)   (int8)
 *   acc    = sum_k code(n,k) * q[m][k] - sum_k q[m][k]   (int32, exact)
 *   y[m][n]= (float)acc * (w_scale / inv_m)              (fp32)
 * The sum of squares is taken in one fixed order, "O256" (256 partial fp32
 * FMA chains, chain j taking the elements k with (k/4) % 256 == j in
 * increasing k; each group of 64 chains 64w..64w+63 reduced by a halving
 * tree (j + 32 into j, then j + 16, ..., j + 1) to g_w; result
 * (g_0 + g_1) + (g_2 + g_3)), so the int8 codes are reproducible.
 *   x:        device fp32 [M][K]; gamma: device fp32 [K]; eps > 0 (the
 *             pages' default is 1e-6) else BL_ERR_INVALID_ARG.
 *   gamma == NULL selects the layer without RMSNorm [HF-38087 "What does
 *             this PR do?": use_rms_norm, off by default]: xn = x, no sum
 *             of squares, and eps is ignored (not validated).
 *   packed_w: device I2_S buffer of W[N][K]; its trailer is not read:
 *             w_scale is the scale (from bitlinear_pack_i2s or
 *             bitlinear_read_scale).
 *   y:        device fp32 [M][N]; every element is written.
 *   workspace: device, >= bitlinear_workspace_bytes(M, K) bytes, 16-byte
 *             aligned, else BL_ERR_WORKSPACE; holds q, inv and qsum after the
 *             call.
 * Asynchronous on `stream`; no host synchronisation. */
bl_status bitlinear_forward(const float *x, const uint8_t *packed_w,
                            float w_scale, const float *gamma, float eps,
                            int64_t M, int64_t K, int64_t N, float *y,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): bitlinear_forward with the same arguments and results but no
 * workspace argument.  The stage results q / inv / qsum go to a scratch
 * array the library holds on each device (BITLINEAR_NOALLOC_SCRATCH_BYTES,
 * allocated with the library's code on that device and held until the
 * process ends) instead of a caller-owned workspace.
 *   bitlinear_workspace_bytes(M, K) > BITLINEAR_NOALLOC_SCRATCH_BYTES ->
 *   BL_ERR_WORKSPACE (e.g. M * K > 16 MiB); the other checks are
 *   bitlinear_forward's.  The scratch array of the current device is used
 *   (the device `stream` belongs to must be current); its address is looked
 *   up on the first call on each device (BL_ERR_HIP if that fails).
 *   Nothing in the scratch array needs to start at zero: each call writes
 *   every q / inv / qsum value it reads.  Every call on a device shares that
 *   device's array, which keeps the last call's contents: calls that may
 *   overlap in time on one device (different streams, or several host
 *   threads without ordering) race and give undefined results; calls on
 *   one stream are ordered and safe.  No hipMalloc / hipFree or other
 *   allocating call is made.  Asynchronous on `stream`. */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES ((size_t)(16u << 20) + (size_t)(64u << 10))
bl_status bitlinear_forward_noalloc(const float *x, const uint8_t *packed_w,
                                    float w_scale, const float *gamma, float eps,
                                    int64_t M, int64_t K, int64_t N, float *y,
                                    void *stream);

/* bitlinear_forward with explicit launch options (NULL = automatic).  For
 * route/launch-shape independence tests and tuning. */
bl_status bitlinear_forward_ex(const float *x, const uint8_t *packed_w,
                               float w_scale, const float *gamma, float eps,
                               int64_t M, int64_t K, int64_t N, float *y,
                               void *workspace, size_t workspace_bytes,
                               const bl_launch *launch, void *stream);

/* One BitLinear forward for bitlinear_forward_batch: the arguments of
 * bitlinear_forward, same meaning and rules. */
typedef struct {
    const float *x;
    const uint8_t *packed_w;
    float w_scale;
    const float *gamma;
    float eps;
    int64_t M, K, N;
    float *y;
    void *workspace;
    size_t workspace_bytes;
} bl_forward_desc;

/* Several independent BitLinear forwards, e.g. the BitLinears of one decoder
 * layer at decode (one launch for the whole layer).  Results are
 * bit-identical to calling bitlinear_forward_ex(descs[i], launch) for each i.
 * The decode-sized ones (M <= 4 with the fused quantisation; automatically,
 * M == 1 with K <= 32768) share one kernel launch per 8.  With the
 * automatic launch shape (and not forced
 * onto the tile route), the others with M <= 8, M * K <= 65536 and
 * K <= 8192 (a few tokens) share one quantisation launch and one one-shot
 * contraction launch per 8, and
 * the prefill-sized ones with K % 256 == 0 and K <= 8192 share one
 * quantisation launch and one tile-kernel launch per 8; the others run one
 * by one.
 *   descs:  HOST array of `count` descriptors (1 <= count <= 64, else
 *           BL_ERR_INVALID_ARG); each is validated as bitlinear_forward
 *           validates its arguments, all before anything is enqueued.
 *   No output (y, workspace) may overlap any input or output of another
 *   descriptor.  Asynchronous on `stream`. */
bl_status bitlinear_forward_batch(const bl_forward_desc *descs, int count,
                                  const bl_launch *launch, void *stream);

/* Stage: RMSNorm + per-row absmax int8 quantisation (the first two steps of
 * bitlinear_forward, bit-identical to them; gamma == NULL: no RMSNorm, eps
 * ignored, as there).
 *   q: device int8 [M][K] (16-byte aligned); inv: device fp32 [M];
 *   qsum: device int32 [M].  Asynchronous on `stream`. */
bl_status bitlinear_act_quant(const float *x, const float *gamma, float eps,
                              int64_t M, int64_t K, int8_t *q, float *inv,
                              int32_t *qsum, void *stream);

/* Stage: the fp32 arithmetic of the normalisation and quantisation scales,
 * elementwise, computed by the same device functions and build as every
 * kernel of the library [HF-38087: r = 1 / sqrt(mean(x^2) + eps) before the
 * absmax int8 quantisation, whose codes depend on r and on the quantisation
 * scale bit for bit].  Exported so that tests can compare the device's
 * square root and division with correctly rounded host arithmetic.
 *   op 0 (BL_FP_SQRT):        out[i] = sqrtf(a[i])               (b unused)
 *   op 1 (BL_FP_DIV):         out[i] = a[i] / b[i]
 *   op 2 (BL_FP_RMS_SCALE):   out[i] = 1 / sqrtf(a[i] / b[i] + eps), with
 *                             b[i] = (float)K, an integer in [1, 2^22]
 *   op 3 (BL_FP_QUANT_SCALE): out[i] = 127 / max(a[i], 1e-5)     (b unused)
 * a, b, out: device fp32 [n] (b may be NULL for ops 0 and 3); n >= 1
 * (BL_ERR_SHAPE otherwise); eps finite (op 2 only).  Unknown op or NULL
 * pointers -> BL_ERR_INVALID_ARG.  Asynchronous on `stream`. */
typedef enum {
    BL_FP_SQRT = 0,
    BL_FP_DIV = 1,
    BL_FP_RMS_SCALE = 2,
    BL_FP_QUANT_SCALE = 3
} bl_fp_op;
bl_status bitlinear_fp32_ops(int op, const float *a, const float *b, float eps, int64_t n,
                             float *out, void *stream);

/* Stage: acc[m][n] = sum_k code(n,k) * q[m][k] - qsum[m] (int32, exact).
 * qsum is taken as given (it is sum_k q[m][k] when it comes from
 * bitlinear_act_quant).  acc: device int32 [M][N].  Asynchronous. */
bl_status bitlinear_matmul_i2s(const int8_t *q, const int32_t *qsum,
                               const uint8_t *packed_w, int64_t M, int64_t K,
                               int64_t N, int32_t *acc, void *stream);

/* bitlinear_matmul_i2s with explicit launch options (NULL = automatic;
 * `fuse` must be -1 or 0). */
bl_status bitlinear_matmul_i2s_ex(const int8_t *q, const int32_t *qsum,
                                  const uint8_t *packed_w, int64_t M,
                                  int64_t K, int64_t N, int32_t *acc,
                                  const bl_launch *launch, void *stream);

/* Activation storage types of bitlinear_forward_io (and weight types of
 * bitlinear_dequant_i2s). */
typedef enum { BL_F32 = 0, BL_BF16 = 1, BL_F16 = 2 } bl_dtype;

/* Dequantisation of an I2_S tensor to a dense float type [CPPB-7,
 * dequantize_row_i2_s, the to_float the BLAS route of the pages runs before
 * a library GEMM]: w_out[n][k] = (code(n,k) - 1) * s in fp32, rounded to
 * w_dtype to nearest with ties to even (BL_F32: bitlinear_unpack_i2s's
 * values).  For comparison with the I2_S path and for callers that run a
 * dense GEMM.  w_out: device [N][K] of w_dtype, 16-byte aligned; an unknown
 * dtype is BL_ERR_INVALID_ARG.  Asynchronous on `stream`. */
bl_status bitlinear_dequant_i2s(const uint8_t *packed, int64_t N, int64_t K, void *w_out,
                                int w_dtype, void *stream);

/* Workspace bytes of bitlinear_forward_io: the forward workspace of (M, K)
 * followed by an int32 accumulator [M][N] (0 if a size is invalid). */
size_t bitlinear_io_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* bitlinear_forward with the activations stored as x_dtype and the output
 * as y_dtype (bl_dtype) [HF-38087 "What does this PR do?": the same layer;
 * the page fixes no storage type].  x is widened exactly to fp32 as it is
 * loaded, the fp32 path runs unchanged (same q, inv, qsum, acc), and
 * y = (float)acc * (w_scale / inv) is rounded to y_dtype to nearest with
 * ties to even (bf16: the high 16 bits of the fp32 word after rounding;
 * fp16: IEEE binary16, overflow to inf).  With both types BL_F32 the bits
 * equal bitlinear_forward's.  One token with K <= 8192 and x_dtype ==
 * y_dtype: one launch (the one-shot decode kernel with the quantisation and
 * the rescale inside) when its workgroups fit on the device at once.
 * Otherwise two launches, the quantisation and a contraction that rounds y
 * in its epilogue, when K <= 8192 and either M <= 8 with M * K <= 65536
 * (the one-shot kernel) or M > 4 with K % 256 == 0 (the tile kernel); else
 * three: quantisation, contraction to the int32 accumulator in the
 * workspace, rescale.
 *   x: device [M][K] of x_dtype; y: device [M][N] of y_dtype; both 16-byte
 *   aligned.  Other arguments and errors as bitlinear_forward; an unknown
 *   dtype is BL_ERR_INVALID_ARG.  workspace: >=
 *   bitlinear_io_workspace_bytes(M, K, N); after the call it holds q, inv
 *   and qsum as bitlinear_forward's does (the accumulator region only on
 *   the three-launch route).  Asynchronous on `stream`. */
bl_status bitlinear_forward_io(const void *x, int x_dtype, const uint8_t *packed_w,
                               float w_scale, const float *gamma, float eps, int64_t M,
                               int64_t K, int64_t N, void *y, int y_dtype, void *workspace,
                               size_t workspace_bytes, void *stream);

/* One forward of bitlinear_forward_io_batch: the arguments of
 * bitlinear_forward_io, same meaning and rules. */
typedef struct {
    const void *x;
    int x_dtype;
    const uint8_t *packed_w;
    float w_scale;
    const float *gamma;
    float eps;
    int64_t M, K, N;
    void *y;
    int y_dtype;
    void *workspace;
    size_t workspace_bytes;
} bl_forward_io_desc;

/* Several independent typed forwards (e.g. a decoder layer's BitLinears
 * with bf16 activations); per descriptor bit-identical to
 * bitlinear_forward_io.  Those with M = 1, K <= 8192 and x_dtype ==
 * y_dtype share one one-shot launch per 8 and per type (quantisation and
 * rescale inside it) when their workgroups fit on the device at once.  The
 * other ones with M <= 8, M * K <= 65536 and K <= 8192 (a few tokens, or
 * one token with x_dtype != y_dtype) share one typed quantisation launch
 * and one one-shot contraction launch (rounding y in its epilogue) per 8
 * of one (x_dtype, y_dtype) pair; the prefill-sized ones (M > 4,
 * K % 256 == 0, K <= 8192) share one typed quantisation launch and one
 * tile-kernel launch per 8 of one pair; the others run as
 * bitlinear_forward_io does.
 *   descs: HOST array, 1 <= count <= 64, each validated as
 *   bitlinear_forward_io validates its arguments, all before anything is
 *   enqueued.  No output (y, workspace) may overlap any input or output of
 *   another descriptor.  Asynchronous on `stream`. */
bl_status bitlinear_forward_io_batch(const bl_forward_io_desc *descs, int count, void *stream);

/* BitNet FFN block [HF-38087, the BitNetMLP excerpt of the review thread:
 * y = down(ffn_sub_norm(act(gate(x)) * up(x))); CPPB-7 summary bullet and
 * the bitnet-b1.58 graph commit: the 2B4T activation is squared ReLU].
 * Each projection is a BitLinear as in bitlinear_forward; the sub-norm is
 * the down projection's own RMSNorm:
 *   g = BitLinear(x; gate, gamma_in), u = BitLinear(x; up, gamma_in)   fp32 [M][F]
 *   a = (max(g, 0) * max(g, 0)) * u                                    fp32 [M][F]
 *   y = BitLinear(a; down, gamma_sub)                                  fp32 [M][H]
 * For F <= 8192, or at M = 1 (F <= 32768), a is never stored: the down
 * projection's quantisation forms it from g and u as it reads them.  At
 * M = 1 the block is two launches (gate and up in one, the down projection
 * with its quantisation in the other); otherwise gate and up take
 * bitlinear_forward_batch's launches and the down projection one
 * quantisation and one contraction launch (for F > 8192, after one
 * elementwise launch that stores a in the workspace).
 *   x: device fp32 [M][H]; y: device fp32 [M][H] (every element written).
 *   packed_gate / packed_up: I2_S of W [F][H]; packed_down: I2_S of W [H][F]
 *             (H and F multiples of 128); s_*: their per-tensor scales.
 *   gamma_in: device fp32 [H] or NULL (no RMSNorm before gate / up);
 *   gamma_sub: device fp32 [F] (the sub-norm's weight) or NULL.
 *   eps: > 0 and finite when either gamma is non-NULL.
 *   workspace: device, >= bitlinear_ffn_workspace_bytes(M, H, F) bytes,
 *             16-byte aligned; after the call it holds g at offset 0 and u
 *             at offset align256(4*M*F) (fp32 [M][F] each), then the three
 *             projections' q / inv / qsum (and a, when F > 8192 and
 *             M > 1); on the
 *             grouped prefill route x is quantised once, into the gate's
 *             part, which both contractions read.
 *   No output may overlap an input.  Errors as bitlinear_forward; all
 *   checks run before anything is enqueued.  Asynchronous on `stream`. */
typedef struct {
    const float *x;
    const float *gamma_in;
    const uint8_t *packed_gate;
    float s_gate;
    const uint8_t *packed_up;
    float s_up;
    const uint8_t *packed_down;
    float s_down;
    const float *gamma_sub;
    float eps;
    int64_t M, H, F;
    float *y;
    void *workspace;
    size_t workspace_bytes;
} bl_ffn_desc;

/* Workspace bytes of bitlinear_ffn_forward (0 if a size is invalid). */
size_t bitlinear_ffn_workspace_bytes(int64_t M, int64_t H, int64_t F);

bl_status bitlinear_ffn_forward(const bl_ffn_desc *desc, void *stream);

/* Calibration probes, used by the benchmark to measure the ceilings the
 * BitLinear kernels are read against; not part of the BitLinear path.
 *   bitlinear_probe_read: one launch that reads `bytes` bytes of `src`
 *     (device, 16-byte aligned, bytes a multiple of 16 and < 2^40) with
 *     coalesced 16-byte loads, all of a thread's loads in flight at once;
 *     sink: device uint32, at least bitlinear_probe_read_sink_words(bytes)
 *     words (one per workgroup, the XOR of what it read).
 *   bitlinear_probe_mfma: `workgroups` workgroups of 256 threads, each wave
 *     issuing `iters` rounds of four independent v_mfma_i32_32x32x32_i8
 *     (2 * 32 * 32 * 32 int ops each); sink: device int32, at least
 *     workgroups * 256 words.  iters >= 1, 1 <= workgroups < 2^31.
 * Errors: BL_ERR_SHAPE for sizes out of range, BL_ERR_INVALID_ARG for NULL
 * pointers or a short sink, BL_ERR_ALIGN for a misaligned src.
 * Asynchronous on `stream`. */
size_t bitlinear_probe_read_sink_words(size_t bytes);
bl_status bitlinear_probe_read(const void *src, size_t bytes, uint32_t *sink, size_t sink_words,
                               void *stream);
bl_status bitlinear_probe_mfma(int64_t iters, int64_t workgroups, int32_t *sink,
                               size_t sink_words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
