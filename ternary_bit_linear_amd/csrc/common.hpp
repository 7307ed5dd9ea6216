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

#include <algorithm>
#include <type_traits>
#include <utility>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockWeights = 128;    // weights per I2_S block
constexpr int kBlockBytes = 32;       // bytes per I2_S block
constexpr int kStepK = 256;           // k per contraction step (two blocks)
constexpr int kStepBytes = 64;        // packed bytes of one row per step
constexpr int kTrailerBytes = 32;
// Dynamic LDS budgets of the decode kernel: q of the fused form (M*K bytes,
// M <= kFuseMaxM) and of the staged form (16 token rows at most).
constexpr int kFuseMaxM = 4;
constexpr int64_t kFuseMaxLds = 32 * 1024;
constexpr int64_t kGemvStageMaxLds = 48 * 1024;

// Codes of field g of a 16-byte packed chunk, one byte per k, as the int8
// MFMA operand.
__device__ __forceinline__ v4i unpack_field(const v4i &p, int g) {
    const int sh = 6 - 2 * g;
    v4i r;
    r.x = (int)(((uint32_t)p.x >> sh) & 0x03030303u);
    r.y = (int)(((uint32_t)p.y >> sh) & 0x03030303u);
    r.z = (int)(((uint32_t)p.z >> sh) & 0x03030303u);
    r.w = (int)(((uint32_t)p.w >> sh) & 0x03030303u);
    return r;
}

// Field g of a 16-byte packed chunk, each code scaled by 2^kFieldShift[g]:
// the code bits are masked where they sit (fields 1..3) or shifted down
// (field 0), 5 instructions per dword instead of 7.  Byte values: field 0 code,
// field 1 16 code, field 2 4 code, field 3 code -- all within int8.  A sum of
// int8 products over field g is then an exact multiple of 2^kFieldShift[g];
// an arithmetic right shift by it restores the sum of codes times
// activations.
constexpr int kFieldShift[4] = {0, 4, 2, 0};
__device__ __forceinline__ v4i unpack_scaled(const v4i &p, int g) {
    v4i r;
    if (g == 0) {
        r.x = (int)(((uint32_t)p.x >> 6) & 0x03030303u);
        r.y = (int)(((uint32_t)p.y >> 6) & 0x03030303u);
        r.z = (int)(((uint32_t)p.z >> 6) & 0x03030303u);
        r.w = (int)(((uint32_t)p.w >> 6) & 0x03030303u);
    } else {
        const uint32_t mask = g == 1 ? 0x30303030u : g == 2 ? 0x0C0C0C0Cu : 0x03030303u;
        r.x = (int)((uint32_t)p.x & mask);
        r.y = (int)((uint32_t)p.y & mask);
        r.z = (int)((uint32_t)p.z & mask);
        r.w = (int)((uint32_t)p.w & mask);
    }
    return r;
}

// D[16][16] += A[16][64] * B[64][16] (int8 -> int32).  Lane l supplies
// A row (l % 16) and B column (l % 16), 16 bytes each for its k-group
// l / 16; D element (i, j) lives in lane j + 16 * (i / 4), register i % 4.
__device__ __forceinline__ v4i mfma16(const v4i &a, const v4i &b, const v4i &c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Range-checked 16-byte loads through a buffer resource: an offset at or
// beyond `bytes` returns zeros (no branch, no clamped address), which is how
// every kernel here handles ragged tiles.  `bytes` must be < 2^31.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // A buffer resource lives in scalar registers.  Every resource built here
    // is wave-uniform; readfirstlane says so to the compiler, which otherwise
    // wraps each load in a loop over lanes whenever a field was computed by
    // a vector instruction.
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t ua = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const int ub = __builtin_amdgcn_readfirstlane((int)bytes);
    // dword3 = 0x00020000: 32-bit data format, the raw-buffer setting on gfx9.
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ua), (short)0, ub, 0x00020000);
}

__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Compile-time index for unrolled rings: f(ic<0>{}), f(ic<1>{}), ...
template <int I>
using ic = std::integral_constant<int, I>;

template <class F, int... I>
__device__ __forceinline__ void unroll_ic(F &&f, std::integer_sequence<int, I...>) {
    (f(ic<I>{}), ...);
}

// Wait until at most VMCNT of this wave's vector-memory loads are
// outstanding (LDS-direct loads included; lgkm and export counters
// untouched).  Scheduling barriers keep every instruction on its side.
template <int VMCNT>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(VMCNT >= 0 && VMCNT < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (VMCNT & 15) | ((VMCNT >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that orders LDS only: waits for this wave's own LDS
// accesses (lgkmcnt(0)) but leaves vector-memory loads in flight, unlike
// __syncthreads, whose fence drains them.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Same with a wave-uniform offset added in the scalar offset field.
__device__ __forceinline__ v4i buf_load16_so(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
}

// 16-byte LDS-direct buffer load: lane i's bytes land at lds + 16 i (lds is
// wave-uniform); an out-of-range offset writes zeros.  Completion is counted
// by vmcnt like any other vector-memory load.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off,
                                               uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds, 16, off, soff, 0, 0);
}

__device__ __forceinline__ float4 buf_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_float4(__int_as_float(v.x), __int_as_float(v.y), __int_as_float(v.z),
                       __int_as_float(v.w));
}

// Activation storage types.  bf16 is carried as its bit pattern; widening
// to fp32 is exact for every type (bf16: the 16 bits become the high half
// of the fp32 word; fp16: f16_low_to_f32 below).
struct bf16_t {
    uint16_t bits;
};
template <typename XT>
constexpr uint32_t kXBytes = sizeof(XT);

// Four consecutive activations at byte offset `off` (out of range: zeros).
template <typename XT>
__device__ __forceinline__ float4 load_x4(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ float4 load_x4<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return buf_load_f4(r, off);
}
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
template <>
__device__ __forceinline__ float4 load_x4<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}
// Hardware widening of one binary16 value held in the low 16 bits of a
// word (v_cvt_f32_f16): exact for every input, subnormals included, as the
// kernels keep fp16 denormals (the default mode).
__device__ __forceinline__ float f16_low_to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
template <>
__device__ __forceinline__ float4 load_x4<_Float16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_float4(f16_low_to_f32(v.x), f16_low_to_f32(v.x >> 16), f16_low_to_f32(v.y),
                       f16_low_to_f32(v.y >> 16));
}

// The same in two parts: the raw words of the four values (out of range:
// zeros), and their widening.  A caller that issues several loads before
// using any widens them only afterwards: a widening placed right behind its
// load makes the compiler wait for that load before the next one goes out.
template <typename XT>
struct XRaw {
    typedef v2u type;  // two words of two half-precision values each
};
template <>
struct XRaw<float> {
    typedef float4 type;
};
template <typename XT>
__device__ __forceinline__ typename XRaw<XT>::type load_x_raw(__amdgpu_buffer_rsrc_t r,
                                                              uint32_t off) {
    if constexpr (std::is_same<XT, float>::value) return buf_load_f4(r, off);
    else return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
template <typename XT>
__device__ __forceinline__ float4 widen_x(const typename XRaw<XT>::type &v) {
    if constexpr (std::is_same<XT, float>::value) {
        return v;
    } else if constexpr (std::is_same<XT, bf16_t>::value) {
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
    } else {
        return make_float4(f16_low_to_f32(v.x), f16_low_to_f32(v.x >> 16), f16_low_to_f32(v.y),
                           f16_low_to_f32(v.y >> 16));
    }
}

// fp32 -> bf16 bits, nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// fp32 -> IEEE binary16 bits, nearest even, by integer operations (exact
// rounding for subnormal results too, whatever the fp16 denormal mode):
// NaN stays a quiet NaN, from 65520 up the result is inf.
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u | ((a >> 13) & 0x3FFu));
    if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520
    if (a >= 0x38800000u) {                                    // >= 2^-14: normal
        const uint32_t r = a - 0x38000000u;                    // rebias 127 -> 15
        return (uint16_t)(sign | ((r + 0xFFFu + ((r >> 13) & 1u)) >> 13));
    }
    // subnormal or zero: units of 2^-24; the scaling is exact, rintf rounds
    // to nearest even (1024 units is the smallest normal, encoded alike)
    const float v = __uint_as_float(a) * 16777216.0f;
    return (uint16_t)(sign | (uint32_t)rintf(v));
}

template <typename YT>
__device__ __forceinline__ uint16_t to_half_bits(float v) {
    if constexpr (std::is_same<YT, bf16_t>::value) return f32_to_bf16_rne(v);
    else return f32_to_f16_rne(v);
}

// One output element of type YT.
template <typename YT>
__device__ __forceinline__ void store_out(YT *y, size_t i, float v) {
    if constexpr (std::is_same<YT, float>::value) y[i] = v;
    else reinterpret_cast<uint16_t *>(y)[i] = to_half_bits<YT>(v);
}

// Halving-tree reduction of the 64 lanes of a wave into lane 0:
// level s = 32, 16, 8, 4, 2, 1 adds lane j + s into lane j (j < s).  Lane
// 0's result is exactly the tree the pinned sum-of-squares order defines.
// Levels 32 and 16 take gfx950's VALU lane swaps, with no LDS round trip:
// v_permlane32_swap(v, v) returns in its second result lanes 32..63 of v in
// lanes 0..31, and v_permlane16_swap(v, v) the odd 16-lane rows in the even
// ones (lanes 16..31 in 0..15).  Levels 8..1 stay inside a 16-lane row (DPP
// row_shl).  Other lanes end with partial values; the result is read with
// readfirstlane (a wave-uniform scalar).
template <class Op>
__device__ __forceinline__ int wave_tree_i(int v, Op op) {
    v = op(v, (int)__builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false)[1]);
    v = op(v, (int)__builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false)[1]);
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x108, 0xF, 0xF, false));  // row_shl:8
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false));  // row_shl:4
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x102, 0xF, 0xF, false));  // row_shl:2
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x101, 0xF, 0xF, false));  // row_shl:1
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ float wave_tree_sum_f(float v) {
    return __int_as_float(wave_tree_i(__float_as_int(v), [](int a, int b) {
        return __float_as_int(__int_as_float(a) + __int_as_float(b));
    }));
}

__device__ __forceinline__ float wave_max(float v) {
    return __int_as_float(wave_tree_i(__float_as_int(v), [](int a, int b) {
        return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
    }));
}

__device__ __forceinline__ int wave_sum_int(int v) {
    return wave_tree_i(v, [](int a, int b) { return a + b; });
}

// RMSNorm scale of a row from its sum of squares (HF-38087: RMSNorm before
// the quantisation, eps inside the root): r = 1 / sqrt(ss / K + eps), with
// IEEE division and square root (the library is built with correctly
// rounded fp32 division and square root, and without fp contraction), so
// the int8 codes that depend on r are the same on any conforming fp32
// implementation.
__device__ __forceinline__ float rms_scale(float ss, int K, float eps) {
    return 1.0f / sqrtf(ss / (float)K + eps);
}

// Quantisation scale of a row from its absolute maximum: 127 / max(amax,
// 1e-5) (IEEE division; the floor only acts on an all-zero row).
__device__ __forceinline__ float quant_scale(float amax) {
    return 127.0f / fmaxf(amax, 1e-5f);
}

// q = clamp(rint(xn * inv), -128, 127).  The clamp never acts, so it is not
// evaluated: |xn| <= amax' = max(amax, 1e-5) and inv = fl(127 / amax') <=
// (127 / amax') (1 + 2^-24), so |fl(xn * inv)| <= 127 (1 + 2^-24)^2 < 127.5
// and rint gives |q| <= 127 (finite inputs; others are unspecified).
__device__ __forceinline__ int quant_one(float xn, float inv) {
    return (int)rintf(xn * inv);
}

__device__ __forceinline__ uint32_t pack_char4(int a, int b, int c, int d) {
    // byte 0 of each: v_perm picks [a0 b0] and [c0 d0], a third joins them
    const uint32_t ab = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0C0C0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Sum of the four signed bytes of a packed word, added to acc (exact).
__device__ __forceinline__ int sum_char4(uint32_t v, int acc) {
    return __builtin_amdgcn_sdot4((int)v, 0x01010101, acc, false);
}

// Arrival counters in LDS.  A wave's LDS operations complete in order, and
// once a wave has waited for its own (lgkmcnt(0)) they are visible to every
// wave of the workgroup; so a wave arrives by waiting for its LDS writes and
// then adding one (lane 0), and a waiting wave polls the counter and issues
// its later LDS reads only after the poll that ends the wait has returned.
// The memory clobbers keep the compiler's LDS writes ahead of the add and
// its later reads behind the poll.  The add and the poll are written as
// instructions because the compiler, unable to tell the counter from the
// LDS targets of weight loads still in flight, would otherwise wait for
// every outstanding global load of the wave first; the poll waits for its
// own result within its statement.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void lds_arrive(int *ctr) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if ((threadIdx.x & 63) == 0)
        asm volatile("ds_add_u32 %0, %1" ::"v"(lds_offset(ctr)), "v"(1) : "memory");
}
__device__ __forceinline__ void lds_wait_count(const int *ctr, int target) {
    const uint32_t a = lds_offset(ctr);
    for (;;) {
        int v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        if (__builtin_amdgcn_readfirstlane(v) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Meeting point of the block form's four waves: a workgroup barrier, or,
// with `spin` set (the four quantising waves of a larger workgroup, whose
// other waves do not take part), an LDS arrival counter: each wave adds one
// per meeting once its own LDS writes are done, then waits until all four
// have (`phase`, kept per wave, is four times the meetings so far).  The
// counter is zero, and visible to the four waves, before their first
// meeting.  The waits end: the four waves are resident in one workgroup and
// each arrives after a bounded amount of work.  Reuse of red[] between
// meetings is safe: a wave writes an entry only after a meeting that every
// wave reaches after its reads of the entry's previous value.
struct QuadSpin {
    int *ctr;
    int phase;
};
__device__ __forceinline__ void quad_meet(QuadSpin *spin) {
    if (!spin) {
        lds_barrier();
        return;
    }
    spin->phase += 4;
    lds_arrive(spin->ctr);
    lds_wait_count(spin->ctr, spin->phase);
}

// Block-wide reductions over exactly 256 threads (4 waves).  `red` is 4
// words of shared memory; the caller's block must reach these uniformly.
// Each takes one barrier (or one quad_meet): a caller that runs several
// reductions gives each its own 4 words (or separates reuses of the same
// words by another barrier), so no trailing barrier is needed.
//
// Sum of squares of one row in the library's fixed order "O256": thread t
// owns the elements k with (k / 4) % 256 == t and accumulates their squares
// with fused multiply-adds in increasing k (its float4 loads at
// k = 4t + 1024 i, in increasing i); the 64 partials of each wave are
// combined by a halving tree (lane j + 32 into j, then j + 16, ... j + 1;
// wave_tree_sum_f); the four wave totals are then added as
// (g0 + g1) + (g2 + g3).
__device__ __forceinline__ float block_sumsq_finish(float p, float *red,
                                                   QuadSpin *spin = nullptr) {
    const int lane = threadIdx.x & 63, wid = (threadIdx.x >> 6) & 3;
    p = wave_tree_sum_f(p);
    if (lane == 0) red[wid] = p;
    quad_meet(spin);
    return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float block_max(float v, float *red, QuadSpin *spin = nullptr) {
    const int lane = threadIdx.x & 63, wid = (threadIdx.x >> 6) & 3;
    v = wave_max(v);
    if (lane == 0) red[wid] = v;
    quad_meet(spin);
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ int block_sum_int(int v, float *red) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    v = wave_sum_int(v);
    int *ri = reinterpret_cast<int *>(red);
    if (lane == 0) ri[wid] = v;
    lds_barrier();
    return ri[0] + ri[1] + ri[2] + ri[3];
}

// Shared-memory words the block reductions of one row take (three
// reductions of 4 words each).
constexpr int kRedWords = 12;

__device__ __forceinline__ float4 xn4(const float4 &x, const float4 &g, float r) {
    return make_float4((x.x * r) * g.x, (x.y * r) * g.y, (x.z * r) * g.z, (x.w * r) * g.w);
}

// gamma == nullptr selects the layer without RMSNorm (HF-38087: use_rms_norm
// off, the activations are quantised as they come): r = 1 and gamma = 1, so
// xn4 returns x exactly.  The gamma descriptor then has no records, so no
// load through it touches memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gamma_rsrc(const float *gamma, int K) {
    return make_rsrc(gamma, gamma ? 4u * (uint32_t)K : 0u);
}
__device__ __forceinline__ float4 gamma_f4(__amdgpu_buffer_rsrc_t rg, uint32_t off, bool norm) {
    return norm ? buf_load_f4(rg, off) : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
}

// Squared-ReLU gated input of the BitNet FFN's down projection
// (HF-38087 BitNetMLP: down(sub_norm(act(gate) * up)); CPPB-7: the 2B4T
// activation is squared ReLU): a = (max(g, 0) * max(g, 0)) * u, in fp32, in
// this order.
__device__ __forceinline__ float relu2_mul(float g, float u) {
    const float r = g > 0.0f ? g : 0.0f;
    return (r * r) * u;
}
__device__ __forceinline__ float4 relu2_mul4(const float4 &g, const float4 &u) {
    return make_float4(relu2_mul(g.x, u.x), relu2_mul(g.y, u.y), relu2_mul(g.z, u.z),
                       relu2_mul(g.w, u.w));
}

// Running max of |v| (exact and order-free for finite values; the chain
// form lets the compiler use three-operand max with abs modifiers).
__device__ __forceinline__ float amax4(float a, const float4 &v) {
    return fmaxf(fmaxf(fmaxf(fmaxf(a, fabsf(v.x)), fabsf(v.y)), fabsf(v.z)), fabsf(v.w));
}

// RMSNorm + absmax int8 quantisation of one token row (HF-38087: RMSNorm on
// the activations before quantisation; the int8 codes and their sum feed the
// I2_S contraction):
//   r = 1 / sqrt(sumsq / K + eps)      (O256 order, IEEE division and root)
//   xn = (x * r) * gamma,  inv = 127 / max(max |xn|, 1e-5)
//   q = clamp(rint(xn * inv), -128, 127),  qsum = sum q.
// With gamma == nullptr there is no RMSNorm: xn = x (no sum of squares).
// GLU: the row is not read from x but formed as relu2_mul(x, u) from the
// gate row x and the up row u (the FFN's down projection input).
// Sink receives store_q(k, 4 packed int8) and store_row(inv, qsum); or, when
// Sink::kDeferSum is true, store_inv(inv) and store_qsum_part(wave, partial)
// (one int per wave of the 256-thread block, written to LDS before the
// caller's next barrier): the activation sum is only needed by the
// contraction's epilogue, so its block reduction (and barrier) is left off
// the path to the first MFMA, and the caller adds the four partials after
// the barrier that publishes q.

// The last step of the block form: inv and the activation sum of the row
// (see kDeferSum above).
template <class Sink>
__device__ __forceinline__ void finish_row(Sink &sink, float inv, int qs, float *red) {
    if constexpr (Sink::kDeferSum) {
        qs = wave_sum_int(qs);
        if ((threadIdx.x & 63) == 0) sink.store_qsum_part((int)(threadIdx.x >> 6) & 3, qs);
        if ((threadIdx.x & 255) == 0) sink.store_inv(inv);
    } else {
        qs = block_sum_int(qs, red + 8);
        if (threadIdx.x == 0) sink.store_row(inv, qs);
    }
}

// Block form (256 threads): thread t owns O256 chain t, i.e. the float4
// groups at k = 4t + 1024 i.  Rows of up to 1024 * CH elements keep x and
// gamma in registers (one global round trip); `issued()` runs once every
// wave of the block has issued those loads (a barrier; with SYNC false, once
// this wave has), so loads the caller issues there queue behind them and do
// not delay the normalisation.  A wave skips the loads of a chunk that lies
// wholly past K.  LONG rows (K > 1024 * CH) are streamed in chunks of CH
// float4 per thread, three times.
// spin: null (the reductions meet at workgroup barriers) or the LDS counter
// on which only the four waves of the block meet (quad_meet; the sink must
// defer the activation sum, whose block form takes a barrier).
template <int CH, bool LONG, bool SYNC = true, bool GLU = false, typename XT = float, class Sink,
          class Hook>
__device__ __forceinline__ void block_act_quant_row(const XT *__restrict__ x,
                                                    const float *__restrict__ gamma,
                                                    float eps, int K, float *red,
                                                    Sink &sink, Hook &&issued,
                                                    const float *__restrict__ u = nullptr,
                                                    QuadSpin *spin = nullptr) {
    static_assert(!GLU || std::is_same<XT, float>::value, "the gated input is fp32");
    constexpr uint32_t XB = kXBytes<XT>;
    const int t4 = 4 * (threadIdx.x & 255);
    constexpr int STRIDE = 1024;
    if constexpr (!LONG) {  // K <= 1024 * CH
        const bool norm = gamma != nullptr;
        const auto rx = make_rsrc(x, XB * (uint32_t)K);
        const auto ru = make_rsrc(u, GLU ? 4u * (uint32_t)K : 0u);
        const auto rg = gamma_rsrc(gamma, K);
        float4 xv[CH], gv[CH], uv[GLU ? CH : 1];
        typename XRaw<XT>::type xr[CH];
        const int wk = 256 * __builtin_amdgcn_readfirstlane(((int)threadIdx.x >> 6) & 3);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int k = t4 + STRIDE * i;
            // Offsets past the row fall outside the resources (exactly K
            // elements each; k and K are multiples of 4), so they read zeros
            // with no select.
            const uint32_t off = 4u * (uint32_t)k;
            // Chunks wholly past K (wave-uniform) are never read below: no
            // load and no initialisation.
            const bool live = STRIDE * i + wk < K;
            // Half-precision words are loaded for every chunk (a chunk past
            // K at an offset outside the resource: zeros), so no branch
            // leaves them to be merged -- the merge would copy them, and
            // wait for each load before the next goes out.
            if constexpr (!std::is_same<XT, float>::value)
                xr[i] = load_x_raw<XT>(rx, live ? XB * (uint32_t)k : kOOB);
            if (live) {
                if constexpr (std::is_same<XT, float>::value)
                    xr[i] = load_x_raw<XT>(rx, XB * (uint32_t)k);
                if constexpr (GLU) uv[i] = buf_load_f4(ru, off);
                gv[i] = gamma_f4(rg, off, norm);
            }
        }
        // Every wave's x / gamma loads are issued before any load the hook
        // issues, so they do not queue behind another wave's weight misses.
        if constexpr (SYNC) __builtin_amdgcn_s_barrier();
        issued();
        // Half-precision x is widened only now, behind every load.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (STRIDE * i + wk < K) xv[i] = widen_x<XT>(xr[i]);
        if constexpr (GLU) {
#pragma unroll
            for (int i = 0; i < CH; ++i)
                if (STRIDE * i + wk < K) xv[i] = relu2_mul4(xv[i], uv[i]);
        }
        // Chunks wholly past K are skipped by the wave (a wave-uniform
        // test); in the others, lanes past K loaded zeros, which leave the
        // sum of squares and the max unchanged.
        float r = 1.0f;
        if (norm) {
            float p = 0.0f;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                if (STRIDE * i + wk < K) {
                    p = __builtin_fmaf(xv[i].x, xv[i].x, p);
                    p = __builtin_fmaf(xv[i].y, xv[i].y, p);
                    p = __builtin_fmaf(xv[i].z, xv[i].z, p);
                    p = __builtin_fmaf(xv[i].w, xv[i].w, p);
                }
            }
            const float ss = block_sumsq_finish(p, red, spin);
            r = rms_scale(ss, K, eps);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (STRIDE * i + wk < K) {
                xv[i] = xn4(xv[i], gv[i], r);  // x is not needed again: keep xn
                amax = amax4(amax, xv[i]);
            }
        }
        amax = block_max(amax, red + 4, spin);
        const float inv = quant_scale(amax);
        int qs = 0;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int k = t4 + STRIDE * i;
            if (k < K) {
                const float4 v = xv[i];
                const int a = quant_one(v.x, inv), b = quant_one(v.y, inv);
                const int c = quant_one(v.z, inv), d = quant_one(v.w, inv);
                const uint32_t w = pack_char4(a, b, c, d);
                qs = sum_char4(w, qs);
                sink.store_q(k, w);
            }
        }
        finish_row(sink, inv, qs, red);
        return;
    } else {
    issued();
    // Long rows: three streamed passes.
    const bool norm = gamma != nullptr;
    const auto rx = make_rsrc(x, XB * (uint32_t)K);
    const auto ru = make_rsrc(u, GLU ? 4u * (uint32_t)K : 0u);
    const auto rg = gamma_rsrc(gamma, K);
    // (offsets past the row read zeros: the resources end at the row)
    auto off_of = [&](int k) -> uint32_t { return 4u * (uint32_t)k; };
    // x of one chunk (GLU: formed from the gate and up rows)
    auto load_x = [&](int k) -> float4 {
        const float4 v = load_x4<XT>(rx, XB * (uint32_t)k);
        if constexpr (GLU) return relu2_mul4(v, buf_load_f4(ru, off_of(k)));
        else return v;
    };
    float r = 1.0f;
    if (norm) {
        float p = 0.0f;
        for (int c0 = 0; c0 < K; c0 += STRIDE * CH) {
            float4 xv[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) xv[i] = load_x(c0 + t4 + STRIDE * i);
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                p = __builtin_fmaf(xv[i].x, xv[i].x, p);
                p = __builtin_fmaf(xv[i].y, xv[i].y, p);
                p = __builtin_fmaf(xv[i].z, xv[i].z, p);
                p = __builtin_fmaf(xv[i].w, xv[i].w, p);
            }
        }
        const float ss = block_sumsq_finish(p, red, spin);
        r = rms_scale(ss, K, eps);
    }
    float amax = 0.0f;
    for (int c0 = 0; c0 < K; c0 += STRIDE * CH) {
        float4 xv[CH], gv[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            xv[i] = load_x(c0 + t4 + STRIDE * i);
            gv[i] = gamma_f4(rg, off_of(c0 + t4 + STRIDE * i), norm);
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) amax = amax4(amax, xn4(xv[i], gv[i], r));
    }
    amax = block_max(amax, red + 4, spin);
    const float inv = quant_scale(amax);
    int qs = 0;
    for (int c0 = 0; c0 < K; c0 += STRIDE * CH) {
        float4 xv[CH], gv[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            xv[i] = load_x(c0 + t4 + STRIDE * i);
            gv[i] = gamma_f4(rg, off_of(c0 + t4 + STRIDE * i), norm);
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int k = c0 + t4 + STRIDE * i;
            if (k < K) {
                const float4 v = xn4(xv[i], gv[i], r);
                const int a = quant_one(v.x, inv), b = quant_one(v.y, inv);
                const int c = quant_one(v.z, inv), d = quant_one(v.w, inv);
                const uint32_t w = pack_char4(a, b, c, d);
                qs = sum_char4(w, qs);
                sink.store_q(k, w);
            }
        }
    }
    finish_row(sink, inv, qs, red);
    }
}

// Barriers block_act_quant_row<..., SYNC = false> takes per row: one per
// block reduction (sum of squares with RMSNorm, max, and the sum of q unless
// the sink defers it).  Waves of a
// larger workgroup that do not run the 256-thread block form call
// block_act_quant_row_barriers instead, so every wave meets the same
// barriers; a change to the block reductions must change both.
__device__ __forceinline__ int block_act_quant_row_barrier_count(bool norm, bool defer_sum) {
    return (norm ? 3 : 2) - (defer_sum ? 1 : 0);
}

// RMSNorm + int8 quantisation of one token row by a 1024-thread workgroup
// with the whole row in registers (rows of up to 4096 * SQ elements), the
// same arithmetic in the same order as the 256-thread block form: O256
// chain t (float4 groups k = 4t + 1024 i) is held by four threads, thread
// 256 h + t holding the groups i in [h SQ, (h + 1) SQ); the chain's sum of
// squares is carried from segment to segment through LDS (one barrier
// each), so every chain is the same sequence of fused multiply-adds, and
// the chain totals are added by the block form's tree.  The maximum and the
// code sum are order-free.  Every wave loads its part of x and gamma at the
// start -- one round trip for the whole row -- then runs `issued()` after a
// barrier, so the loads the caller issues there queue behind all of them.
// q goes to q (LDS; not with TO_LDS false) and, when gq is set, to global
// memory; inv to *inv (and *ginv); the per-wave code sums to qpart[16].
// GLU: the row is relu2_mul(x, u) of the gate row x and the up row u (the
// FFN's down projection input), formed as they arrive; gamma is then loaded
// after the product (it is first needed after the sum of squares), so that
// x, u and gamma are never all held at once.
template <int SQ, bool GLU = false, bool TO_LDS = true, class Hook>
__device__ __forceinline__ void wide_act_quant_row(const float *__restrict__ x,
                                                   const float *__restrict__ gamma, float eps,
                                                   int K, float *red, float *chain, int8_t *q,
                                                   int8_t *gq, float *inv, float *ginv, int *qpart,
                                                   Hook &&issued,
                                                   const float *__restrict__ u = nullptr) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int h = __builtin_amdgcn_readfirstlane(wid >> 2);  // segment of the chain
    const int t = tid & 255;                                  // chain
    const int ni = (K + 1023) / 1024;                         // float4 groups per chain
    const bool norm = gamma != nullptr;
    const auto rx = make_rsrc(x, 4u * (uint32_t)K);
    const auto ru = make_rsrc(u, GLU ? 4u * (uint32_t)K : 0u);
    const auto rg = gamma_rsrc(gamma, K);
    float4 xv[SQ], gv[SQ];
    auto off_of = [&](int i) { return 4u * (uint32_t)(4 * t + 1024 * (h * SQ + i)); };
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
        if (h * SQ + i < ni) {  // wave-uniform; lanes past K read zeros
            xv[i] = load_x4<float>(rx, off_of(i));
            gv[i] = GLU ? buf_load_f4(ru, off_of(i)) : gamma_f4(rg, off_of(i), norm);
        } else {
            xv[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            gv[i] = xv[i];
        }
    }
    __builtin_amdgcn_s_barrier();
    issued();
    if constexpr (GLU) {
        // x <- relu2_mul(x, u), then gamma into the registers u held
#pragma unroll
        for (int i = 0; i < SQ; ++i) {
            xv[i] = relu2_mul4(xv[i], gv[i]);
            gv[i] = h * SQ + i < ni ? gamma_f4(rg, off_of(i), norm)
                                    : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
    float r = 1.0f;
    if (norm) {
        float p = 0.0f;
        for (int s = 0; s < 4; ++s) {
            if (h == s) {
                if (s > 0) p = chain[t];
#pragma unroll
                for (int i = 0; i < SQ; ++i) {
                    if (h * SQ + i < ni) {
                        p = __builtin_fmaf(xv[i].x, xv[i].x, p);
                        p = __builtin_fmaf(xv[i].y, xv[i].y, p);
                        p = __builtin_fmaf(xv[i].z, xv[i].z, p);
                        p = __builtin_fmaf(xv[i].w, xv[i].w, p);
                    }
                }
                if (s < 3) chain[t] = p;
            }
            if (s < 3) lds_barrier();
        }
        // Segment 3 holds the chain totals: waves 12..15 are the block
        // form's four waves.
        if (h == 3) {
            p = wave_tree_sum_f(p);
            if (lane == 0) red[wid - 12] = p;
        }
        lds_barrier();
        r = rms_scale((red[0] + red[1]) + (red[2] + red[3]), K, eps);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
        xv[i] = xn4(xv[i], gv[i], r);
        amax = amax4(amax, xv[i]);
    }
    amax = wave_max(amax);
    if (lane == 0) red[4 + wid] = amax;
    lds_barrier();
    float m = red[4];
#pragma unroll
    for (int w = 1; w < 16; ++w) m = fmaxf(m, red[4 + w]);
    const float iv = quant_scale(m);
    int qs = 0;
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
        const int k = 4 * t + 1024 * (h * SQ + i);
        if (k < K) {
            const float4 v = xv[i];
            const uint32_t w = pack_char4(quant_one(v.x, iv), quant_one(v.y, iv),
                                          quant_one(v.z, iv), quant_one(v.w, iv));
            qs = sum_char4(w, qs);
            if constexpr (TO_LDS) *reinterpret_cast<uint32_t *>(q + k) = w;
            if (gq) *reinterpret_cast<uint32_t *>(gq + k) = w;
        }
    }
    qs = wave_sum_int(qs);
    if (lane == 0) qpart[wid] = qs;
    if (tid == 0) {
        *inv = iv;
        if (gq) *ginv = iv;
    }
}
__device__ __forceinline__ void block_act_quant_row_barriers(bool norm, bool defer_sum) {
    const int n = block_act_quant_row_barrier_count(norm, defer_sum);
    for (int i = 0; i < n; ++i) lds_barrier();
}

// Wave form (64 threads, no LDS, no barrier): lane j owns the four O256
// chains j, 64 + j, 128 + j, 192 + j, i.e. the float4 groups at
// k = 1024 i + 256 w + 4 j (w = 0..3).  Each chain group w is reduced by the
// same halving tree (wave_tree_sum_f) and the four totals are added as
// (g0 + g1) + (g2 + g3) -- the same bits as the block form.  Rows of up to
// 1024 * CI elements stay in registers; longer rows take three passes.
template <int CI, typename XT = float, class Sink>
__device__ __forceinline__ void wave_act_quant_row(const XT *__restrict__ x,
                                                   const float *__restrict__ gamma,
                                                   float eps, int K, Sink &sink) {
    constexpr uint32_t XB = kXBytes<XT>;
    const int lane = threadIdx.x & 63;
    const bool norm = gamma != nullptr;
    const auto rx = make_rsrc(x, XB * (uint32_t)K);
    const auto rg = gamma_rsrc(gamma, K);
    // (offsets past the row read zeros: the resources end at the row)
    auto off_of = [&](int k) -> uint32_t { return 4u * (uint32_t)k; };
    auto xoff_of = [&](int k) -> uint32_t { return XB * (uint32_t)k; };
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool in_regs = K <= 1024 * CI;
    float4 xv[CI][4], gv[CI][4];
    for (int c0 = 0; c0 < K; c0 += 1024 * CI) {
#pragma unroll
        for (int i = 0; i < CI; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int k = c0 + 1024 * i + 256 * w + 4 * lane;
                const uint32_t off = off_of(k);
                xv[i][w] = load_x4<XT>(rx, xoff_of(k));
                if (in_regs) gv[i][w] = gamma_f4(rg, off, norm);
            }
#pragma unroll
        for (int i = 0; i < CI; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                p[w] = __builtin_fmaf(xv[i][w].x, xv[i][w].x, p[w]);
                p[w] = __builtin_fmaf(xv[i][w].y, xv[i][w].y, p[w]);
                p[w] = __builtin_fmaf(xv[i][w].z, xv[i][w].z, p[w]);
                p[w] = __builtin_fmaf(xv[i][w].w, xv[i][w].w, p[w]);
            }
    }
    float r = 1.0f;
    if (norm) {
#pragma unroll
        for (int w = 0; w < 4; ++w) p[w] = wave_tree_sum_f(p[w]);
        const float ss = (p[0] + p[1]) + (p[2] + p[3]);
        r = rms_scale(ss, K, eps);
    }
    float amax = 0.0f;
    for (int c0 = 0; c0 < K; c0 += 1024 * CI) {
        if (!in_regs) {
#pragma unroll
            for (int i = 0; i < CI; ++i)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int k = c0 + 1024 * i + 256 * w + 4 * lane;
                    const uint32_t off = off_of(k);
                    xv[i][w] = load_x4<XT>(rx, xoff_of(k));
                    gv[i][w] = gamma_f4(rg, off, norm);
                }
        }
#pragma unroll
        for (int i = 0; i < CI; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) amax = amax4(amax, xn4(xv[i][w], gv[i][w], r));
    }
    amax = wave_max(amax);
    const float inv = quant_scale(amax);
    int qs = 0;
    for (int c0 = 0; c0 < K; c0 += 1024 * CI) {
        if (!in_regs) {
#pragma unroll
            for (int i = 0; i < CI; ++i)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int k = c0 + 1024 * i + 256 * w + 4 * lane;
                    const uint32_t off = off_of(k);
                    xv[i][w] = load_x4<XT>(rx, xoff_of(k));
                    gv[i][w] = gamma_f4(rg, off, norm);
                }
        }
#pragma unroll
        for (int i = 0; i < CI; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int k = c0 + 1024 * i + 256 * w + 4 * lane;
                if (k < K) {
                    const float4 v = xn4(xv[i][w], gv[i][w], r);
                    const int a = quant_one(v.x, inv), b = quant_one(v.y, inv);
                    const int c = quant_one(v.z, inv), d = quant_one(v.w, inv);
                    const uint32_t w = pack_char4(a, b, c, d);
                    qs = sum_char4(w, qs);
                    sink.store_q(k, w);
                }
            }
    }
    qs = wave_sum_int(qs);
    if (lane == 0) sink.store_row(inv, qs);
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

// Quantisation of the FFN down projection's input relu2_mul(g, u) (rows of
// g and u: [M][K], gamma the sub-norm or nullptr); same codes as
// launch_act_quant over that product.
hipError_t launch_act_quant_glu(const float *g, const float *u, const float *gamma, float eps,
                                int64_t M, int64_t K, int8_t *q, float *inv, int32_t *qsum,
                                hipStream_t s);

// Activation I/O types of the typed forward (the values of bl_dtype).
constexpr int kIoF32 = 0, kIoBf16 = 1, kIoF16 = 2;

// launch_act_quant over x stored as xtype (widened to fp32 on load; the
// same codes as launch_act_quant over the widened values).
hipError_t launch_act_quant_io(const void *x, int xtype, const float *gamma, float eps, int64_t M,
                               int64_t K, int8_t *q, float *inv, int32_t *qsum, hipStream_t s);

// y = (float)acc * (w_scale / inv[m]) stored as ytype (rounded to nearest
// even).
hipError_t launch_rescale_io(const int32_t *acc, const float *inv, float w_scale, int64_t M,
                             int64_t N, void *y, int ytype, hipStream_t s);

// Elementwise fp32 arithmetic of the normalisation and quantisation (op 0
// sqrtf(a), 1 a / b, 2 rms_scale(a, (int)b, eps), 3 quant_scale(a)), for
// checking it against host arithmetic.
hipError_t launch_fp32_ops(int op, const float *a, const float *b, float eps, int64_t n,
                           float *out, hipStream_t s);

// a = relu2_mul(g, u) elementwise over n floats (n % 4 == 0, 16-byte
// aligned arrays).
hipError_t launch_relu2_mul(const float *g, const float *u, float *a, int64_t n, hipStream_t s);



// Batched quantisation: up to 8 independent (x, gamma, eps, M, K) with
// K <= 8192 each, one launch, bit-identical to launch_act_quant per problem.
struct ActQuantDesc {
    const void *x;  // of type io (widened to fp32 as it is loaded)
    const float *gamma;
    float eps;
    int64_t M, K;
    int8_t *q;
    float *inv;
    int32_t *qsum;
    int io = 0;     // kIoF32 / kIoBf16 / kIoF16; one type per launch
};
constexpr int64_t kActQuantBatchMaxK = 8192;
hipError_t launch_act_quant_batch(const ActQuantDesc *d, int count, hipStream_t s);

// Decode route, separate quantisation (q / inv / qsum already computed):
// tokens in groups of 16 on int8 MFMA 16x16x64.  With y != NULL the
// epilogue writes y = (acc - qsum) * (w_scale / inv); otherwise it writes
// acc - qsum to `acc`.  `variant` 0 picks a launch shape from K.
hipError_t launch_gemv(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M, int64_t K, int64_t N,
                       float *y, int32_t *acc, int variant, hipStream_t s);

// Decode route with the RMSNorm + quantisation fused in (M <= kFuseMaxM,
// M*K <= kFuseMaxLds): every workgroup recomputes q from x, gamma, eps; the
// first workgroup of each problem also writes q / inv / qsum.  One launch
// serves `count` (<= 8) independent problems.
struct FusedDecode {
    const float *x;
    const float *gamma;
    const uint8_t *packed;
    float *y;
    int8_t *q;
    float *inv;
    int32_t *qsum;
    float eps;
    float w_scale;
    int64_t M, K, N;
    // Non-null: the input row is relu2_mul(x, u) (the FFN's down projection
    // over the gate rows x and up rows u).  One-shot route with M == 1 only;
    // every problem of a launch has it or none does.
    const float *u = nullptr;
    // Storage type of x and y (kIoF32 / kIoBf16 / kIoF16; x and y point to
    // that type).  Half types: one-shot route, M == 1, K <= 8192, no GLU,
    // one type per launch.
    int io = 0;
};
hipError_t launch_gemv_fused(const FusedDecode *d, int count, int variant, hipStream_t s);

// One-shot decode contraction of up to 8 problems in one launch, int8
// activations in global memory (M <= 8, M*K <= kShotMaxQ, K <= 32768).
// y (rescaled) when every y is non-null, else acc (int32).
constexpr int64_t kShotMaxQ = 64 * 1024;
constexpr int64_t kShotFusedMaxQ = 32 * 1024;  // fused form: x rows in registers
// Automatic one-shot choice for a single contraction (the range it was
// measured on); batches take blocks up to kShotMaxQ through the batched pair.
constexpr int64_t kShotSingleMaxQ = 32 * 1024;
struct ShotDecode {
    const int8_t *q;
    const float *inv;
    const int32_t *qsum;
    const uint8_t *packed;
    float *y;       // of type io (y != nullptr), else acc
    int32_t *acc;
    float w_scale;
    int64_t M, K, N;
    int io = 0;     // kIoF32 / kIoBf16 / kIoF16: one type per launch
};
// shape: 1..shot_num_shapes() asks for that launch shape (taken when every
// problem fits it), 0 picks one.
int shot_num_shapes();
constexpr int kShotShapeCount = 8;  // shot_num_shapes()
// Rounds of workgroups the device needs for these problems in the one-shot
// form with its own choice of launch shape (INT64_MAX: not supported).  One
// round means every workgroup is resident at once.  glu: fused, over the
// gated FFN input (u set).
int64_t shot_rounds(const int64_t *M, const int64_t *K, const int64_t *N, int count, bool fused,
                    bool glu = false);
bool shot_supported(int64_t M, int64_t K);
hipError_t launch_gemv_shot(const ShotDecode *d, int count, int shape, hipStream_t s);
// The same with the RMSNorm + quantisation fused in (M <= kFuseMaxM): every
// workgroup normalises its problem's rows while its weight loads are in
// flight; the first workgroup of each problem also writes q / inv / qsum.
bool shot_fused_supported(int64_t M, int64_t K);
hipError_t launch_gemv_shot_fused(const FusedDecode *d, int count, int shape, hipStream_t s);
// A few tokens (up to kFewFusedMaxM) with the quantisation fused in: the
// one-shot launch shape whose workgroups quantise their rows in parallel
// groups of four waves.  Whether every problem has M <= kFewFusedMaxM rows
// of K <= 8192 (in registers) and that shape holds the set in one round.
constexpr int64_t kFewFusedMaxM = 3;
constexpr int kFewFusedShapeVariant = 8;  // the `shape` launch_gemv_shot_fused takes for it
bool few_fused_one_round(const int64_t *M, const int64_t *K, const int64_t *N, int count);
// Rolling form of the one-shot contraction (each wave streams its weights
// through a small register ring), for problem sets the device does not hold
// in one round: q from global memory (M <= 8, M * K <= kShotMaxQ), or fused
// for one token per problem (fp32 x / y; all problems of a launch with the
// gated FFN input u, or none).
bool roll_supported(int64_t M, int64_t K);
hipError_t launch_gemv_roll(const ShotDecode *d, int count, hipStream_t s);
bool roll_fused_supported(int64_t M, int64_t K);
hipError_t launch_gemv_roll_fused(const FusedDecode *d, int count, hipStream_t s);
// One-shot launch of up to 8 problems with q from global memory where all
// of its workgroups are resident at once, else the rolling form where it
// applies (measured faster), else the one-shot form over several rounds.
hipError_t launch_gemv_shot_auto(const ShotDecode *d, int count, hipStream_t s);
int gemv_num_variants();

// Prefill route (activation tiles staged in LDS, int8 MFMA).  Same
// epilogue convention as launch_gemv.
hipError_t launch_gemm(const int8_t *q, const float *inv, const int32_t *qsum,
                       const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, int64_t N, float *y, int32_t *acc,
                       int variant, hipStream_t s);
int gemm_num_variants();

// Grouped prefill launch: up to 8 independent contractions (K % 256 == 0
// each; all with y, or all with acc) in one launch, bit-identical to
// launch_gemm per problem.
struct GemmDesc {
    const int8_t *q;
    const float *inv;
    const int32_t *qsum;
    const uint8_t *packed;
    float w_scale;
    int64_t M, K, N;
    float *y;    // of type io (rounded to nearest even) when not fp32
    int32_t *acc;
    int io = 0;  // kIoF32 / kIoBf16 / kIoF16; one type per launch
};
bool gemm_group_supported(int64_t K);
hipError_t launch_gemm_group(const GemmDesc *d, int count, hipStream_t s);

// Prefill route on the 32 x 32 x 32 int8 MFMA (activations and packed
// weights staged through LDS rings, one I2_S block per step): up to 8
// problems (any K % 128 == 0) in one launch, bit-identical to launch_gemm.
// shape: 1..gemm32_num_shapes() (0 picks the first).
int gemm32_num_shapes();
hipError_t launch_gemm32_group(const GemmDesc *d, int count, int shape, hipStream_t s);
// Whether the automatic choice takes the 32 x 32 x 32 kernel for a group.
bool gemm32_preferred(const GemmDesc *d, int count);

// Compute units of the current device (looked up once per device).
int device_cus();

// Calibration probes: one pass reading `bytes` (a multiple of 16; one
// sink word per workgroup, probe_read_blocks(bytes) of them), and `blocks`
// workgroups of back-to-back int8 MFMAs (256 sink words each).
int64_t probe_read_blocks(uint64_t bytes);
hipError_t launch_probe_read(const uint8_t *src, uint64_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_mfma(int64_t iters, int64_t blocks, int32_t *sink, hipStream_t s);

// I2_S packing: scan (codes + magnitude statistics into the trailer words),
// then finalize (trailer = scale + 28 zero bytes).
hipError_t launch_pack_scan(const float *w, int64_t N, int64_t K,
                            uint8_t *packed, hipStream_t s);
hipError_t launch_pack_init(uint8_t *trailer, hipStream_t s);
hipError_t launch_pack_finalize(uint8_t *trailer, float scale, hipStream_t s);
// Dequantisation to wtype (kIoF32 / kIoBf16 / kIoF16): (code - 1) * scale,
// rounded to nearest even for the half types.
hipError_t launch_dequant(const uint8_t *packed, int64_t N, int64_t K, void *w, int wtype,
                          hipStream_t s);
hipError_t launch_unpack(const uint8_t *packed, int64_t N, int64_t K,
                         float *w, hipStream_t s);

}  // namespace bl
