/*
 * oracle.c -- plain, slow CPU oracle of the ternary BitLinear forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file.  It is used by tests/, by the smoke check and by
 * the CPU-baseline leg of the benchmark, and by nothing else.  It shares no
 * code, header, table or helper with the HIP library; it was written from
 * the pages' description of the method, not from the GPU code.
 *
 * Sources (web pages, cited by title and section):
 *   [HF-38087]  huggingface/transformers PR #38087, "Add optional RMSNorm
 *               support to BitNet quantization (config + layers)", section
 *               "What does this PR do?" (use_rms_norm, rms_norm_eps = 1e-6,
 *               RMSNorm applied to the activations before quantisation).
 *   [CPPB-7]    eejd/cpp-bitnet PR #7, "fix: I2_S ARM kernel layout +
 *               squared-ReLU FFN": the summary bullets (I2_S NEON kernel;
 *               llama-quantize I2_S), section "Known gaps", and the commit
 *               messages "ggml-cpu: I2_S NEON kernel ... calling conventions"
 *               and "llama-quantize I2_S emits the canonical layout".
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *   - I2_S block: 128 weights in 32 bytes; weight j of a block lives in byte
 *     j % 32, 2-bit field j / 32; field g occupies bits (7-2g)..(6-2g).  The
 *     pages give the block size, the word "interleaved" and the wrong
 *     (sequential: byte i/4, field i%4) layout; the field-to-bit order is a
 *     reading ("parity unpinned" by the pages).
 *   - code = w/scale + 1, i.e. -1 -> 0, 0 -> 1, +1 -> 2; the activation sum is
 *     subtracted from sum(code*q) so the result is sum((code-1)*q).
 *   - scale = the first non-zero |w| in row-major order; the input must be
 *     ternary x scale; the 32-byte trailer holds the fp32 scale (little
 *     endian) and 28 zero bytes; row length K must be a multiple of 128.
 *   - RMSNorm: xn = (x * r) * gamma with r = 1 / sqrt(sum(x^2)/K + eps), in
 *     fp32 with correctly rounded division and square root.  The sum of
 *     squares uses one pinned order, "O256", defined at oracle_sumsq.
 *   - int8 quantisation: per token, inv = 127 / max(amax, 1e-5),
 *     q = clamp(round-half-even(xn * inv), -128, 127), qsum = sum(q).
 *   - y = acc * (w_scale / inv), computed here in fp64 from the exact int32
 *     accumulator.
 *   - use_rms_norm off (gamma NULL): the activations are quantised as they
 *     come, with no RMSNorm.
 *   - FFN block: each projection is a BitLinear; the sub-norm is the down
 *     projection's RMSNorm; the gate/up outputs are fp32 values
 *     (float)acc * (w_scale / inv) and a = (relu(g) * relu(g)) * u in fp32,
 *     so the down projection's int8 codes are decided from the same fp32
 *     values the product computes.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -shared
 * -fPIC.  The fp32 steps must not be contracted or reassociated: they decide
 * integer codes.  OpenMP only splits independent rows; it does not change
 * any arithmetic order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status values (the oracle's own; the product library defines its own). */
#define ORC_OK 0
#define ORC_ERR_SHAPE 2
#define ORC_ERR_NOT_TERNARY 4

#define ORC_BLOCK_WEIGHTS 128 /* weights per I2_S block            [CPPB-7] */
#define ORC_BLOCK_BYTES 32    /* bytes per I2_S block (4 codes/B)  [CPPB-7] */
#define ORC_TRAILER_BYTES 32  /* scale + 28 zero bytes             [CPPB-7] */

int oracle_version(void) { return 1; }

int64_t oracle_packed_bytes(int64_t N, int64_t K) {
    return N * K / 4 + ORC_TRAILER_BYTES;
}

/* Position of weight (n, k) inside the packed buffer: the byte index and the
 * right-shift that brings its 2-bit field to bits 1..0.  Within a 128-weight
 * block, weight j sits in byte j % 32 and field j / 32; field 0 is the most
 * significant bit pair.  [CPPB-7, commit "llama-quantize I2_S emits the
 * canonical layout" and the NEON-kernel commit: 128-weight / 32-byte
 * interleaved blocks, not byte i/4 field i%4.] */
static void i2s_position(int64_t K, int64_t n, int64_t k, int64_t *byte_index,
                         int *shift) {
    int64_t block = k / ORC_BLOCK_WEIGHTS;
    int64_t j = k % ORC_BLOCK_WEIGHTS;
    int64_t field = j / 32;
    *byte_index = n * (K / 4) + block * ORC_BLOCK_BYTES + (j % 32);
    *shift = 6 - 2 * (int)field;
}

static uint32_t float_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* I2_S packer [CPPB-7, summary bullet "llama-quantize I2_S emits the canonical
 * layout" and section "Known gaps"]: one call per tensor, scale = first
 * non-zero |w| (row-major), input must be ternary x scale, row length a
 * multiple of 128, trailer = scale + 28 zero bytes.
 * w: fp32 [N][K] row-major.  out: N*K/4 + 32 bytes.  scale_out: may be NULL.
 * Returns ORC_ERR_SHAPE if K % 128 != 0 or a size is < 1, ORC_ERR_NOT_TERNARY
 * if a non-zero magnitude differs from the first one or a value is not
 * finite (out is then unspecified). */
int oracle_pack_i2s(const float *w, int64_t N, int64_t K, uint8_t *out,
                    float *scale_out) {
    if (N < 1 || K < 1 || K % ORC_BLOCK_WEIGHTS != 0) return ORC_ERR_SHAPE;
    const int64_t total = N * K;

    /* 1. scale = |first non-zero| (-0.0 counts as zero). */
    float scale = 0.0f;
    for (int64_t i = 0; i < total; ++i) {
        if (w[i] != 0.0f || isnan(w[i])) {
            scale = fabsf(w[i]);
            break;
        }
    }
    /* 2. the input must be ternary x scale: every value finite and every
     *    non-zero magnitude bitwise equal to the scale. */
    for (int64_t i = 0; i < total; ++i) {
        if (!isfinite(w[i])) return ORC_ERR_NOT_TERNARY;
        if (w[i] != 0.0f && float_bits(fabsf(w[i])) != float_bits(scale))
            return ORC_ERR_NOT_TERNARY;
    }
    /* 3. codes: w / scale is -1, 0 or +1; stored code is that plus one. */
    memset(out, 0, (size_t)(total / 4));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            float v = w[n * K + k];
            int code = (v > 0.0f) ? 2 : (v < 0.0f) ? 0 : 1;
            int64_t b;
            int sh;
            i2s_position(K, n, k, &b, &sh);
            out[b] = (uint8_t)(out[b] | (code << sh));
        }
    }
    /* 4. trailer: fp32 scale, little endian, then 28 zero bytes. */
    uint8_t *tr = out + total / 4;
    uint32_t sb = float_bits(scale);
    tr[0] = (uint8_t)(sb & 0xff);
    tr[1] = (uint8_t)((sb >> 8) & 0xff);
    tr[2] = (uint8_t)((sb >> 16) & 0xff);
    tr[3] = (uint8_t)((sb >> 24) & 0xff);
    memset(tr + 4, 0, ORC_TRAILER_BYTES - 4);
    if (scale_out) *scale_out = scale;
    return ORC_OK;
}

/* Stored 2-bit code of weight (n, k). */
int oracle_code_at(const uint8_t *packed, int64_t K, int64_t n, int64_t k) {
    int64_t b;
    int sh;
    i2s_position(K, n, k, &b, &sh);
    return (packed[b] >> sh) & 3;
}

/* Scale read back from the trailer. */
float oracle_read_scale(const uint8_t *packed, int64_t N, int64_t K) {
    const uint8_t *tr = packed + N * K / 4;
    uint32_t sb = (uint32_t)tr[0] | ((uint32_t)tr[1] << 8) |
                  ((uint32_t)tr[2] << 16) | ((uint32_t)tr[3] << 24);
    float s;
    memcpy(&s, &sb, sizeof s);
    return s;
}

/* Unpacker, the to_float direction [CPPB-7, NEON-kernel commit: the layout
 * read by dequantize_row_i2_s]: w = (code - 1) * scale. */
int oracle_unpack_i2s(const uint8_t *packed, int64_t N, int64_t K, float *w) {
    if (N < 1 || K < 1 || K % ORC_BLOCK_WEIGHTS != 0) return ORC_ERR_SHAPE;
    float s = oracle_read_scale(packed, N, K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            w[n * K + k] = (float)(oracle_code_at(packed, K, n, k) - 1) * s;
    return ORC_OK;
}

/* Sum of squares of one row in the pinned fp32 order "O256" (the pages fix
 * no order; one is needed because the result decides integer codes):
 *   256 partial sums p[0..255], all +0.0f;
 *   for k = 0, 1, ..., K-1: p[(k/4) % 256] = fmaf(v[k], v[k], p[(k/4) % 256]);
 *   each group of 64 partials p[64w .. 64w+63] (w = 0..3) is halved:
 *     for s = 32, 16, 8, 4, 2, 1: p[64w+j] = p[64w+j] + p[64w+j+s] for j < s,
 *   giving g[w] = p[64w];
 *   result (g[0] + g[1]) + (g[2] + g[3]). */
float oracle_sumsq(const float *v, int64_t K) {
    float p[256];
    for (int j = 0; j < 256; ++j) p[j] = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        int j = (int)((k / 4) % 256);
        p[j] = fmaf(v[k], v[k], p[j]);
    }
    float g[4];
    for (int w = 0; w < 4; ++w) {
        float *q = p + 64 * w;
        for (int s = 32; s >= 1; s /= 2)
            for (int j = 0; j < s; ++j) q[j] = q[j] + q[j + s];
        g[w] = q[0];
    }
    return (g[0] + g[1]) + (g[2] + g[3]);
}

/* RMSNorm of one token row, fp32 [HF-38087, "What does this PR do?": the
 * BitNet RMSNorm, eps default 1e-6, applied to activations before
 * quantisation]: r = 1 / sqrt(sumsq / K + eps); xn = (x * r) * gamma. */
static void rmsnorm_row(const float *x, const float *gamma, float eps,
                        int64_t K, float *xn) {
    float ss = oracle_sumsq(x, K);
    float ms = ss / (float)K;
    float r = 1.0f / sqrtf(ms + eps);
    for (int64_t k = 0; k < K; ++k) xn[k] = (x[k] * r) * gamma[k];
}

int oracle_rmsnorm(const float *x, const float *gamma, float eps, int64_t M,
                   int64_t K, float *xn) {
    if (M < 1 || K < 1) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) rmsnorm_row(x + m * K, gamma, eps, K, xn + m * K);
    return ORC_OK;
}

/* Per-token absmax int8 quantisation of the normalised row (the "i8" operand
 * of the i2 x i8 dot product, [CPPB-7, NEON-kernel commit]; the activation
 * sum is kept for the code offset):
 *   amax = max |xn|; inv = 127 / max(amax, 1e-5);
 *   q = clamp(rint(xn * inv), -128, 127) with round-half-to-even;
 *   qsum = sum q.  xn_scratch holds K floats per row.
 * gamma == NULL is the layer without RMSNorm [HF-38087, "What does this PR
 * do?": use_rms_norm, off by default]: xn = x and eps is not used. */
int oracle_act_quant(const float *x, const float *gamma, float eps, int64_t M,
                     int64_t K, int8_t *q, float *inv, int32_t *qsum,
                     float *xn_scratch) {
    if (M < 1 || K < 1) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float *xn = xn_scratch + m * K;
        if (gamma)
            rmsnorm_row(x + m * K, gamma, eps, K, xn);
        else
            for (int64_t k = 0; k < K; ++k) xn[k] = x[m * K + k];
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xn[k]);
            if (a > amax) amax = a;
        }
        float iv = 127.0f / fmaxf(amax, 1e-5f);
        int32_t sum = 0;
        for (int64_t k = 0; k < K; ++k) {
            float t = rintf(xn[k] * iv);
            if (t > 127.0f) t = 127.0f;
            if (t < -128.0f) t = -128.0f;
            int8_t v = (int8_t)t;
            q[m * K + k] = v;
            sum += v;
        }
        inv[m] = iv;
        qsum[m] = sum;
    }
    return ORC_OK;
}

/* Ternary x int8 contraction over the packed codes, with the activation-sum
 * offset [CPPB-7, NEON-kernel commit: codes are not -1/0/+1, the caller
 * subtracts the activation sum]:
 *   acc[m][n] = sum_k code(n, k) * q[m][k] - qsum[m]     (exact int32).
 * W is [N][K] (rows of the packed buffer), y = x W^T. */
int oracle_matmul_i2s(const int8_t *q, const int32_t *qsum,
                      const uint8_t *packed, int64_t M, int64_t K, int64_t N,
                      int32_t *acc) {
    if (M < 1 || N < 1 || K < 1 || K % ORC_BLOCK_WEIGHTS != 0) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)oracle_code_at(packed, K, n, k) * q[m * K + k];
            acc[m * N + n] = (int32_t)(s - qsum[m]);
        }
    }
    return ORC_OK;
}

/* Rescale back to float: y = acc * (w_scale / inv[m]), evaluated in fp64 from
 * the exact integer accumulator. */
int oracle_rescale(const int32_t *acc, const float *inv, float w_scale,
                   int64_t M, int64_t N, double *y) {
    if (M < 1 || N < 1) return ORC_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * ((double)w_scale / (double)inv[m]);
    return ORC_OK;
}

/* The whole forward: RMSNorm -> int8 quantisation -> ternary contraction ->
 * rescale.  Scratch buffers are the caller's: xn (M*K floats), q (M*K),
 * inv (M), qsum (M), acc (M*N). */
int oracle_forward(const float *x, const uint8_t *packed, float w_scale,
                   const float *gamma, float eps, int64_t M, int64_t K,
                   int64_t N, double *y, float *xn, int8_t *q, float *inv,
                   int32_t *qsum, int32_t *acc) {
    int st = oracle_act_quant(x, gamma, eps, M, K, q, inv, qsum, xn);
    if (st) return st;
    st = oracle_matmul_i2s(q, qsum, packed, M, K, N, acc);
    if (st) return st;
    return oracle_rescale(acc, inv, w_scale, M, N, y);
}

/* BitLinear output in fp32, the precision the product returns it in:
 * y32 = (float)acc * (w_scale / inv[m]), one IEEE division and one
 * multiplication.  Used where a BitLinear output feeds another step whose
 * integer codes depend on it (the FFN block below), so that both sides take
 * those decisions from the same fp32 values. */
int oracle_rescale_f32(const int32_t *acc, const float *inv, float w_scale,
                       int64_t M, int64_t N, float *y) {
    if (M < 1 || N < 1) return ORC_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m) {
        const float c = w_scale / inv[m];
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = (float)acc[m * N + n] * c;
    }
    return ORC_OK;
}

/* One BitLinear with fp32 output (act_quant -> contraction -> rescale_f32);
 * gamma NULL: no RMSNorm.  Scratch is allocated here. */
static int bitlinear_f32(const float *x, const float *gamma, float eps, int64_t M,
                         int64_t K, int64_t N, const uint8_t *packed, float w_scale,
                         float *y) {
    float *xn = malloc(sizeof(float) * (size_t)(M * K));
    int8_t *q = malloc((size_t)(M * K));
    float *inv = malloc(sizeof(float) * (size_t)M);
    int32_t *qsum = malloc(sizeof(int32_t) * (size_t)M);
    int32_t *acc = malloc(sizeof(int32_t) * (size_t)(M * N));
    int st = ORC_ERR_SHAPE;
    if (xn && q && inv && qsum && acc) {
        st = oracle_act_quant(x, gamma, eps, M, K, q, inv, qsum, xn);
        if (!st) st = oracle_matmul_i2s(q, qsum, packed, M, K, N, acc);
        if (!st) st = oracle_rescale_f32(acc, inv, w_scale, M, N, y);
    }
    free(xn); free(q); free(inv); free(qsum); free(acc);
    return st;
}

/* Squared-ReLU gate of the FFN block [CPPB-7 summary bullet: the 2B4T
 * activation is relu2; HF-38087 BitNetMLP: act(gate) * up]:
 * a = (max(g, 0) * max(g, 0)) * u, element by element, fp32, this order. */
int oracle_relu2_mul(const float *g, const float *u, int64_t n, float *a) {
    if (n < 1) return ORC_ERR_SHAPE;
    for (int64_t i = 0; i < n; ++i) {
        const float r = g[i] > 0.0f ? g[i] : 0.0f;
        a[i] = (r * r) * u[i];
    }
    return ORC_OK;
}

/* BitNet FFN block [HF-38087, the BitNetMLP excerpt in the review thread:
 * down(ffn_sub_norm(act(gate(x)) * up(x))); CPPB-7 summary bullet and the
 * commit on the bitnet-b1.58 graph: the 2B4T activation is squared ReLU,
 * not SiLU].  Every projection is a BitLinear (RMSNorm with its gamma, or
 * none when the gamma is NULL, then int8 quantisation and the ternary
 * contraction); the sub-norm is the down projection's own RMSNorm:
 *   g = BitLinear(x; gate, gamma_in)      [M][F] fp32
 *   u = BitLinear(x; up,   gamma_in)      [M][F] fp32
 *   a = (max(g, 0) * max(g, 0)) * u       [M][F] fp32, this order
 *   y = BitLinear(a; down, gamma_sub)     [M][H] fp64 (oracle_forward's rescale)
 * Shapes: x [M][H]; gate, up packed from [F][H]; down packed from [H][F];
 * gamma_in [H], gamma_sub [F].  g, u, a are returned for inspection. */
int oracle_ffn(const float *x, const float *gamma_in, float eps, int64_t M, int64_t H,
               int64_t F, const uint8_t *p_gate, float s_gate, const uint8_t *p_up,
               float s_up, const uint8_t *p_down, float s_down, const float *gamma_sub,
               float *g, float *u, float *a, double *y) {
    if (M < 1 || H < 1 || F < 1 || H % ORC_BLOCK_WEIGHTS || F % ORC_BLOCK_WEIGHTS)
        return ORC_ERR_SHAPE;
    int st = bitlinear_f32(x, gamma_in, eps, M, H, F, p_gate, s_gate, g);
    if (!st) st = bitlinear_f32(x, gamma_in, eps, M, H, F, p_up, s_up, u);
    if (st) return st;
    oracle_relu2_mul(g, u, M * F, a);
    float *xn = malloc(sizeof(float) * (size_t)(M * F));
    int8_t *q = malloc((size_t)(M * F));
    float *inv = malloc(sizeof(float) * (size_t)M);
    int32_t *qsum = malloc(sizeof(int32_t) * (size_t)M);
    int32_t *acc = malloc(sizeof(int32_t) * (size_t)(M * H));
    st = ORC_ERR_SHAPE;
    if (xn && q && inv && qsum && acc)
        st = oracle_forward(a, p_down, s_down, gamma_sub, eps, M, F, H, y, xn, q, inv, qsum, acc);
    free(xn); free(q); free(inv); free(qsum); free(acc);
    return st;
}

/* bf16 <-> fp32 for the bf16 activation I/O variant (the pages fix no
 * half-precision format; the reading is the IEEE-style bfloat16: the top 16
 * bits of an fp32, rounded to nearest with ties to even).
 *   to fp32: exact (the 16 bits become the high half of the fp32 word).
 *   from fp32: round to nearest even on the 16 dropped bits; NaN stays a
 *   quiet NaN with its sign. */
int oracle_bf16_to_f32(const uint16_t *in, int64_t n, float *out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)in[i] << 16;
        memcpy(out + i, &u, 4);
    }
    return ORC_OK;
}

int oracle_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = float_bits(in[i]);
        if ((u & 0x7fffffffu) > 0x7f800000u) {
            out[i] = (uint16_t)((u >> 16) | 0x0040u);
            continue;
        }
        const uint32_t lsb = (u >> 16) & 1u;
        u += 0x7fffu + lsb;
        out[i] = (uint16_t)(u >> 16);
    }
    return ORC_OK;
}
