// Shared device helpers for the gfx950 MoE kernels: bf16 conversion, MFMA
// operand types and the LDS tile swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- bounds checks of the MOE_DEBUG build.  A kernel checks each global
// address it forms from indices against the extent of the buffer it must
// lie in: an access outside is counted (with the source line of the first
// one, per translation unit) and redirected to the buffer's first byte, so
// a wrong index becomes a recorded violation rather than a memory fault or a
// silent overwrite.  moe_debug_bounds (include/moe_debug.h) reads and clears
// the record.  In release builds MOE_CHECKED(p, ...) is p itself.
#ifdef MOE_DEBUG
static __device__ uint32_t moe_oob[2];   // violations, source line of the first
template <typename T>
__device__ __forceinline__ T *checked(T *p, size_t n, const void *base, size_t bytes, int line) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), lo = reinterpret_cast<uintptr_t>(base);
    if (base && a >= lo && a + n <= lo + bytes) return p;
    if (atomicAdd(&moe_oob[0], 1u) == 0u) moe_oob[1] = (uint32_t)line;
    return reinterpret_cast<T *>(reinterpret_cast<uintptr_t>(base));
}
#define MOE_CHECKED(p, n, base, bytes) ::moe::checked((p), (size_t)(n), (const void *)(base), (size_t)(bytes), __LINE__)
// Host side: this translation unit's record into rec[2], cleared after.
#define MOE_DEBUG_READER(fn)                                                       \
    hipError_t fn(uint32_t *rec) {                                                 \
        hipError_t e = hipMemcpyFromSymbol(rec, HIP_SYMBOL(moe_oob), 8);           \
        const uint32_t zero[2] = {0u, 0u};                                         \
        return e == hipSuccess ? hipMemcpyToSymbol(HIP_SYMBOL(moe_oob), zero, 8) : e; \
    }
#else
#define MOE_CHECKED(p, n, base, bytes) (p)
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return b >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two bf16 values packed low/high in a 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// A tile row holds 64 bf16 (128 bytes = 8 chunks of 16 bytes).  The chunk
// index is XORed with the low three bits of the row.  Measured on gfx950
// (SQ_LDS_BANK_CONFLICT) for the MFMA fragment read -- lane l reads chunk
// 4*kk + l/16 of row 16*m + l%16 with ds_read_b128 -- this layout has no
// bank conflicts (so does XOR with (row >> 1) & 7), while XOR with
// (row ^ row >> 3) & 7 costs 4 extra cycles per read and no swizzle 12.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// Swizzle of a tile with K-step BK (rows of BK bf16).  Rows of 32 bf16
// (64 bytes = 4 chunks) measured the same way: XOR with (row >> 1) & 3 is
// conflict-free; XOR with row & 3, (row >> 2) & 3 or none cost 4 extra cycles.
// Rows of 128 bf16 (256 bytes = 16 chunks): XOR with row & 15 is
// conflict-free; XOR with row & 7 or (row >> 1) & 7 costs one extra cycle
// per read, none seven.  Rows of 256 bf16 (512 bytes, 16-row token tiles of
// the 4-bit weight path) take the same XOR with row & 15: a fragment read
// touches 16 rows, whose chunks then fall in 16 different 16-byte slots of
// every 256 bytes, as for 256-byte rows.
template <int BK>
__device__ __forceinline__ int tswz(int row, int chunk) {
    if constexpr (BK == 128 || BK == 256) return chunk ^ (row & 15);
    else if constexpr (BK == 64) return chunk ^ (row & 7);
    else return chunk ^ ((row >> 1) & 3);
}

// 16x16x128 MFMA on MXFP4 (E2M1) operands with per-lane E8M0 block scales,
// fp32 accumulation.  Lane l supplies row l % 16 and K values 32*(l/16) ..
// +31 as 16 bytes of codes (two per byte, the even K index in the low
// nibble) plus that block's scale byte; the result layout is that of
// mfma16x16x32 (checked on gfx950 against a plain host loop).
typedef int i32x8 __attribute__((ext_vector_type(8)));
// The scale bytes are byte SA of scale_a and byte SB of scale_b (the
// instruction's own byte select, so a register can hold four scales).
template <int SA, int SB>
__device__ __forceinline__ f32x4 mfma_fp4x128(const u32x4 &a, const u32x4 &b, f32x4 c, uint32_t scale_a,
                                              uint32_t scale_b) {
    const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, SA, (int)scale_a, SB, (int)scale_b);
}

// The same with the byte selects as arguments; in unrolled loops they are
// constants and the switch folds away.
__device__ __forceinline__ f32x4 mfma_fp4x128(const u32x4 &a, const u32x4 &b, f32x4 c, uint32_t scale_a,
                                              uint32_t scale_b, int sa, int sb) {
#define MOE_FP4_CASE(x, y) \
    case 4 * x + y: return mfma_fp4x128<x, y>(a, b, c, scale_a, scale_b);
    switch (4 * sa + sb) {
        MOE_FP4_CASE(0, 0) MOE_FP4_CASE(0, 1) MOE_FP4_CASE(0, 2) MOE_FP4_CASE(0, 3)
        MOE_FP4_CASE(1, 0) MOE_FP4_CASE(1, 1) MOE_FP4_CASE(1, 2) MOE_FP4_CASE(1, 3)
        MOE_FP4_CASE(2, 0) MOE_FP4_CASE(2, 1) MOE_FP4_CASE(2, 2) MOE_FP4_CASE(2, 3)
        MOE_FP4_CASE(3, 0) MOE_FP4_CASE(3, 1) MOE_FP4_CASE(3, 2)
        default: return mfma_fp4x128<3, 3>(a, b, c, scale_a, scale_b);
    }
#undef MOE_FP4_CASE
}

// FP8 E4M3 code (the low byte of b) -> fp32 (OCP 8-bit floating point:
// exponent bias 7, three mantissa bits, exponent field 0 subnormal m * 2^-9,
// no infinities) in one v_cvt_f32_fp8, which on gfx950 decodes the OCP
// encoding (all 254 finite codes checked bitwise against a host decode).  The
// NaN codes S.1111.111 are not valid scales; they give NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8(b, 0); }

// Eight E2M1 codes (a 32-bit word, the lower K index in the low nibble)
// times an fp32 factor, as eight bf16 values in K order.  Each code goes to
// fp32 exactly, is multiplied in fp32 and rounded to bf16; for an E4M3 factor
// the product has at most 6 significant bits, so the rounding is exact.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int Q>   // codes 2Q and 2Q + 1 (byte Q)
__device__ __forceinline__ uint32_t e2m1x2_times_scale(uint32_t codes, float s) {
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, Q);
    const bf16x2_t b = {(__bf16)(v[0] * s), (__bf16)(v[1] * s)};
    return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ u32x4 e2m1x8_times_scale(uint32_t codes, float s) {
    return u32x4{e2m1x2_times_scale<0>(codes, s), e2m1x2_times_scale<1>(codes, s),
                 e2m1x2_times_scale<2>(codes, s), e2m1x2_times_scale<3>(codes, s)};
}

// 16x16x32 bf16 MFMA with fp32 accumulation.  Operand layout per lane l:
// A row (l % 16), k = 8*(l/16) .. +7; B column (l % 16), same k range;
// result rows 4*(l/16) + r (r = 0..3), column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, f32x4 c) {
    bf16x8 av = __builtin_bit_cast(bf16x8, a);
    bf16x8 bv = __builtin_bit_cast(bf16x8, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// gelu_pytorch_tanh: 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated as z / (1 + exp(-2u)) (the same function: 0.5 (1 + tanh u) is
// the logistic function of 2u).  Large |u| saturates to z or -0.
__device__ __forceinline__ float gelu_tanh(float z) {
    const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
    const float k1 = 0.044715f;
    float u = k0 * (z + k1 * z * z * z);
    return __fdividef(z, 1.0f + __expf(-2.0f * u));
}

// One 16-byte output chunk of the weighted combine: out[t][c..c+7] =
// (sum_s y_sh32[s][t][c..c+7], if given) + sum_{j<k} w[t*k+j] * y[r_j][c..c+7]
// with r_j = inv[t*k+j] (y in expert order) or t*k+j (inv == nullptr: y in
// (token, slot) order, so the row loads need no index load first): fp32
// adds over s in order, then fp32 fmas in ascending j, one bf16 rounding.
// Each y row is read exactly once, so its loads carry the non-temporal hint
// (Zipf-skewed 8192 tokens: 81 -> 78 us).
__device__ __forceinline__ void combine_chunk(const uint16_t *__restrict__ y, const int32_t *__restrict__ inv,
                                              const float *__restrict__ w, const float *__restrict__ y_sh32,
                                              int nsplit, uint16_t *__restrict__ out, int t, int c, int T, int H,
                                              int k) {
    const int32_t *ti = inv ? inv + (size_t)t * k : nullptr;
    const float *tw = w + (size_t)t * k;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int sp = 0; y_sh32 && sp < nsplit; ++sp) {
        const float *r = MOE_CHECKED(y_sh32 + ((size_t)sp * T + t) * H + c, 32, y_sh32, (size_t)nsplit * T * H * 4);
        const f32x4 a = *reinterpret_cast<const f32x4 *>(r), b = *reinterpret_cast<const f32x4 *>(r + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[q] += a[q];
            acc[4 + q] += b[q];
        }
    }
    for (int j0 = 0; j0 < k; j0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = min(j0 + u, k - 1);
            const size_t row = ti ? (size_t)ti[j] : (size_t)t * k + j;
            v[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(MOE_CHECKED(y + row * H + c, 16, y, (size_t)T * k * H * 2)));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u >= k) break;
            const float wj = tw[j0 + u];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(wj, bf16_to_f32(v[u][q] & 0xFFFFu), acc[2 * q]);
                acc[2 * q + 1] = fmaf(wj, bf16_to_f32(v[u][q] >> 16), acc[2 * q + 1]);
            }
        }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *reinterpret_cast<u32x4 *>(MOE_CHECKED(out + (size_t)t * H + c, 16, out, (size_t)T * H * 2)) = o;
}

}  // namespace moe
