// common.hpp -- device helpers shared by the gfx950 kernels of the ternary
// BitLinear library, and the host-side launch interface between the source
// files.  Nothing here is exported from the shared library.
//
// I2_S layout [eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout +
// squared-ReLU FFN", NEON-kernel and quantizer commits]: a 128-weight block
// of a row is 32 bytes; weight j of the block is in byte j % 32, 2-bit field
// j / 32, field g in bits (7-2g)..(6-2g).  Stored code = w/scale + 1.
//
// Register layout used by every contraction kernel here.  A 16-byte load of
// row bytes [16h, 16h+16) of a block (h = 0, 1) holds, for each field g, the
// codes of 16 consecutive k: 128*block + 32g + 16h + [0, 16).  One such load
// therefore feeds four int8 MFMAs (one per field), each lane supplying 16
// consecutive k -- the per-lane operand width of v_mfma_i32_16x16x64_i8.
// The activation operand of each lane is the 16 int8 q values at the same k,
// so the hardware's k order inside a lane never matters: A and B use the
// same lane/byte -> k map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockWeights = 128;    // weights per I2_S block
constexpr int kBlockBytes = 32;       // bytes per I2_S block
constexpr int kStepK = 256;           // k per contraction step (two blocks)
constexpr int kStepBytes = 64;        // packed bytes of one row per step
constexpr int kTrailerBytes = 32;

// Codes of field g of a 16-byte packed chunk, one byte per k, as the int8
// MFMA operand.
__device__ __forceinline__ v4i unpack_field(const uint4 &p, int g) {
    const int sh = 6 - 2 * g;
    v4i r;
    r.x = (int)((p.x >> sh) & 0x03030303u);
    r.y = (int)((p.y >> sh) & 0x03030303u);
    r.z = (int)((p.z >> sh) & 0x03030303u);
    r.w = (int)((p.w >> sh) & 0x03030303u);
    return r;
}

// D[16][16] += A[16][64] * B[64][16] (int8 -> int32).  Lane l supplies
// A row (l % 16) and B column (l % 16), 16 bytes each for its k-group
// l / 16; D element (i, j) lives in lane j + 16 * (i / 4), register i % 4.
__device__ __forceinline__ v4i mfma16(const v4i &a, const v4i &b, const v4i &c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Sum of squares of one row in the library's fixed order: lane j of a wave
// owns the elements k with (k / 4) % 64 == j and accumulates them with
// fused multiply-adds in increasing k; the 64 partial sums are then combined
// by a halving tree (j + 32 into j, then j + 16 into j, ... then j + 1 into
// j).  The xor butterfly below evaluates exactly that tree; every lane ends
// with the same value.
__device__ __forceinline__ float wave_sumsq(const float *__restrict__ row, int K, int lane) {
    float p = 0.0f;
    for (int k = 4 * lane; k < K; k += 4 * kWave) {
        const float4 v = *reinterpret_cast<const float4 *>(row + k);
        p = __builtin_fmaf(v.x, v.x, p);
        p = __builtin_fmaf(v.y, v.y, p);
        p = __builtin_fmaf(v.z, v.z, p);
        p = __builtin_fmaf(v.w, v.w, p);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_xor(p, s, kWave);
    return p;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, kWave));
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, kWave);
    return v;
}

__device__ __forceinline__ int quant_one(float xn, float inv) {
    float t = rintf(xn * inv);
    t = fminf(fmaxf(t, -128.0f), 127.0f);
    return (int)t;
}

__device__ __forceinline__ uint32_t pack_char4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) |
           ((uint32_t)(c & 0xff) << 16) | ((uint32_t)(d & 0xff) << 24);
}

// RMSNorm + absmax int8 quantisation of `rows` (<= 4) consecutive token rows
// by a block of NT threads (NT = 256 or 512).  Wave w < rows computes the sum
// of squares of row w in the fixed order; then the whole block computes, per
// row, amax of xn = (x * r) * gamma, inv = 127 / max(amax, 1e-5), and
// q = clamp(rint(xn * inv), -128, 127) with qsum = sum q.  Sink receives
// store_q(row, k, packed 4 x int8) and store_row(row, inv, qsum).
// `red` is >= 2 * NT / 64 floats of shared memory; the block must call this
// uniformly.
template <int NT, class Sink>
__device__ __forceinline__ void block_act_quant(const float *__restrict__ x,
                                                const float *__restrict__ gamma,
                                                float eps, int rows, int K,
                                                float *red, Sink &sink) {
    constexpr int NW = NT / kWave;
    static_assert(NW >= 4 && NW <= 8, "block_act_quant: 256 or 512 threads");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    __shared__ float r_sh[4];
    if (wid < rows) {
        const float ss = wave_sumsq(x + (size_t)wid * K, K, lane);
        const float ms = ss / (float)K;
        const float r = 1.0f / sqrtf(ms + eps);
        if (lane == 0) r_sh[wid] = r;
    }
    __syncthreads();
    for (int m = 0; m < rows; ++m) {
        const float r = r_sh[m];
        const float *xr = x + (size_t)m * K;
        float amax = 0.0f;
        for (int k = 4 * tid; k < K; k += 4 * NT) {
            const float4 v = *reinterpret_cast<const float4 *>(xr + k);
            const float4 g = *reinterpret_cast<const float4 *>(gamma + k);
            amax = fmaxf(amax, fabsf((v.x * r) * g.x));
            amax = fmaxf(amax, fabsf((v.y * r) * g.y));
            amax = fmaxf(amax, fabsf((v.z * r) * g.z));
            amax = fmaxf(amax, fabsf((v.w * r) * g.w));
        }
        amax = wave_max(amax);
        if (lane == 0) red[wid] = amax;
        __syncthreads();
        amax = red[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) amax = fmaxf(amax, red[w]);
        const float inv = 127.0f / fmaxf(amax, 1e-5f);
        int qs = 0;
        for (int k = 4 * tid; k < K; k += 4 * NT) {
            const float4 v = *reinterpret_cast<const float4 *>(xr + k);
            const float4 g = *reinterpret_cast<const float4 *>(gamma + k);
            const int a = quant_one((v.x * r) * g.x, inv);
            const int b = quant_one((v.y * r) * g.y, inv);
            const int c = quant_one((v.z * r) * g.z, inv);
            const int d = quant_one((v.w * r) * g.w, inv);
            qs += a + b + c + d;
            sink.store_q(m, k, pack_char4(a, b, c, d));
        }
        qs = wave_sum_int(qs);
        if (lane == 0) reinterpret_cast<int *>(red)[NW + wid] = qs;
        __syncthreads();
        if (tid == 0) {
            const int *ri = reinterpret_cast<const int *>(red) + NW;
            int total = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) total += ri[w];
            sink.store_row(m, inv, total);
        }
        __syncthreads();
    }
}

}  // namespace bl

// ---------------------------------------------------------------------------
// Host-side launch interface between the library's source files.  Every
// function enqueues on `s` and returns the launch status; arguments have
// been validated by the caller.
namespace bl {

hipError_t launch_act_quant(const float *x, const float *gamma, float eps,
                            int64_t M, int64_t K, int8_t *q, float *inv,
                            int32_t *qsum, hipStream_t s);

// Decode route (tokens in groups of 16, int8 MFMA 16x16x64).  With y != NULL
// the epilogue writes y = (acc - qsum) * (w_scale / inv); otherwise it writes
// acc - qsum to `acc`.  With fused = true, q/inv/qsum are recomputed in
// every workgroup from x, gamma, eps (M <= 4, M*K bytes of LDS) and
// workgroup 0 writes them to q/inv/qsum (which are then outputs).
hipError_t launch_gemv(const float *x, const float *gamma, float eps,
                       const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, int64_t N, float *y, int32_t *acc,
                       bool fused, int variant, hipStream_t s);
int gemv_num_variants();

// Prefill route (activation tiles staged in LDS, int8 MFMA).  Same
// epilogue convention as launch_gemv.
hipError_t launch_gemm(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, int64_t N, float *y, int32_t *acc,
                       int variant, hipStream_t s);
int gemm_num_variants();

// I2_S packing: scan (codes + magnitude statistics into the trailer words),
// then finalize (trailer = scale + 28 zero bytes).
hipError_t launch_pack_scan(const float *w, int64_t N, int64_t K,
                            uint8_t *packed, hipStream_t s);
hipError_t launch_pack_init(uint8_t *trailer, hipStream_t s);
hipError_t launch_pack_finalize(uint8_t *trailer, float scale, hipStream_t s);
hipError_t launch_unpack(const uint8_t *packed, int64_t N, int64_t K,
                         float *w, hipStream_t s);

}  // namespace bl
