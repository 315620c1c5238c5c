// MXFP4 quantisation of bf16 rows, per 32 consecutive values along a row
// (OCP Microscaling Formats v1.0 conversion; the W4A4 checkpoints of this
// model are named by the vLLM-Ascend Gemma4 tutorial, section 3.1): the
// block's scale is 2^e with e = floor(log2 amax) - 2 (clamped to [-127,
// 127]; 0 for an all-zero block), stored as the E8M0 byte e + 127; every
// value v becomes the E2M1 code nearest to v / 2^e, ties to the even code,
// saturating at 6, with v's own sign bit.  Two codes per byte, the even
// index in the low nibble.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// floor(log2 |v|) of a non-zero bf16 magnitude (15-bit pattern, sign cleared).
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
    const int expf = (int)(mag >> 7);
    if (expf > 0) return expf - 127;
    return (31 - __builtin_clz(mag)) - 133;   // subnormal: mantissa m, value m * 2^-133
}

// E2M1 magnitude code of m >= 0 (round to nearest, ties to the even code).
// At a tie the comparison that decides it is strict when the lower code is
// even and inclusive when the upper one is.
__device__ __forceinline__ uint32_t e2m1_code(float m) {
    return (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) + (uint32_t)(m >= 1.75f) +
           (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
}

// One thread per 32-value block.
__global__ __launch_bounds__(256) void quantize_mx_kernel(const uint16_t *__restrict__ src, long long nblocks,
                                                         int K, uint8_t *__restrict__ codes,
                                                         uint8_t *__restrict__ scales) {
    const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const int bpr = K / 32;
    const long long row = b / bpr;
    const int blk = (int)(b % bpr);
    const u32x4 *p = reinterpret_cast<const u32x4 *>(
        MOE_CHECKED(src + row * K + blk * 32, 64, src, (size_t)nblocks * 64));
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p[i];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) amax = max(amax, max(v[i][q] & 0x7FFFu, (v[i][q] >> 16) & 0x7FFFu));
    int e = amax == 0 ? 0 : bf16_floor_log2(amax) - 2;
    e = min(max(e, -127), 127);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, a normal float for |e| <= 126...
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t bits = (v[i][q] >> (16 * h)) & 0xFFFFu;
                const float m = bf16_to_f32(bits & 0x7FFFu) * inv;
                const uint32_t code = e2m1_code(m) | ((bits >> 12) & 8u);
                word |= code << (4 * (2 * q + h));
            }
        }
        out[i] = word;
    }
    *reinterpret_cast<u32x4 *>(MOE_CHECKED(codes + row * (K / 2) + blk * 16, 16, codes, (size_t)nblocks * 16)) = out;
    *MOE_CHECKED(scales + row * bpr + blk, 1, scales, (size_t)nblocks) = (uint8_t)(e + 127);
}

// NVFP4 quantisation of bf16 rows, per 16 consecutive values, relative to
// the tensor's fp32 input scale g (the Gemma-4-26B-A4B-NVFP4 verification
// report, section 2.3: 4-bit float activations in groups of 16).  In fp32:
// s = amax / (6 g) goes to the nearest E4M3 value (ties to the even code,
// 448 from 448 up), step = that scale * g, and each value v to the E2M1 code
// nearest to v / step (ties to the even code, saturating at 6, v's sign
// bit); a block whose scale is 0 gets zero codes.  Outputs: codes [rows][K/2]
// (even index in the low nibble) and E4M3 scale codes [rows][K/16], and/or
// the decoded values without g, E2M1 x scale, as bf16 (exact: at most six
// significant bits), which the bf16 matrix cores multiply.

// Nearest E4M3 value of s >= 0 (OCP 8-bit floating point: exponent bias 7,
// three mantissa bits, subnormals m * 2^-9, largest finite 448): with e the
// binade of s (at least -6, the subnormal range), s / 2^(e-3) rounded half
// to even and scaled back; both scalings are exact, and an even rounded
// mantissa is an even code.
__device__ __forceinline__ float e4m3_nearest(float s) {
    if (!(s < 448.0f)) return 448.0f;
    const int E = (int)((__float_as_uint(s) >> 23) & 0xFFu) - 127;
    const int e = E < -6 ? -6 : E;
    const float up = __uint_as_float((uint32_t)(127 + 3 - e) << 23);     // 2^(3-e), normal for e >= -6
    const float down = __uint_as_float((uint32_t)(127 - 3 + e) << 23);   // 2^(e-3)
    return rintf(s * up) * down;
}

// E4M3 code of a value produced by e4m3_nearest (non-negative, on the grid).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    if (v < 0.015625f) return (uint32_t)(v * 512.0f);                   // subnormal: m * 2^-9
    const uint32_t b = __float_as_uint(v);
    return ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);       // exponent + 7, three mantissa bits
}

__device__ __forceinline__ float e2m1_magnitude(uint32_t c) {
    // 0, 0.5, 1, 1.5, 2, 3, 4, 6
    return c < 4 ? 0.5f * (float)c : (float)(c < 6 ? c - 2 : 2 * c - 8);
}

// One thread per 16-value block.
// (src and dq may be the same rows: each thread reads its block before it
// writes it, and no other thread touches it.)
__global__ __launch_bounds__(256) void quantize_nv_kernel(const uint16_t *src, long long nblocks, int K,
                                                         const float *__restrict__ g_ptr,
                                                         uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                         uint16_t *dq) {
    const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const int bpr = K / 16;
    const long long row = b / bpr;
    const int blk = (int)(b % bpr);
    const u32x4 *p = reinterpret_cast<const u32x4 *>(
        MOE_CHECKED(src + row * K + blk * 16, 32, src, (size_t)nblocks * 32));
    const u32x4 v[2] = {p[0], p[1]};
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) amax = max(amax, max(v[i][q] & 0x7FFFu, (v[i][q] >> 16) & 0x7FFFu));
    const float g = *g_ptr;
    const float s = bf16_to_f32(amax) / (6.0f * g);
    const float sq = e4m3_nearest(s);
    const float step = sq * g;
    uint32_t cw[2] = {0u, 0u};
    uint32_t dw[8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t pair = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t bits = (v[i][q] >> (16 * h)) & 0xFFFFu;
                const uint32_t sign = (bits >> 15) & 1u;
                uint32_t mag = 0;
                if (step > 0.0f) mag = e2m1_code(bf16_to_f32(bits & 0x7FFFu) / step);
                const uint32_t code = step > 0.0f ? (mag | (sign << 3)) : 0u;
                cw[i] |= code << (4 * (2 * q + h));
                // decoded value without g: E2M1 x scale, exact in bf16
                const uint32_t val = __float_as_uint(e2m1_magnitude(code & 7u) * sq) >> 16;
                pair |= (val | ((code >> 3) << 15)) << (16 * h);
            }
            dw[4 * i + q] = pair;
        }
    if (codes) {
        *reinterpret_cast<uint2 *>(MOE_CHECKED(codes + row * (K / 2) + blk * 8, 8, codes, (size_t)nblocks * 8)) =
            make_uint2(cw[0], cw[1]);
        *MOE_CHECKED(scales + row * bpr + blk, 1, scales, (size_t)nblocks) = (uint8_t)e4m3_code(sq);
    }
    if (dq) {
        u32x4 *o = reinterpret_cast<u32x4 *>(MOE_CHECKED(dq + row * K + blk * 16, 32, dq, (size_t)nblocks * 32));
        o[0] = u32x4{dw[0], dw[1], dw[2], dw[3]};
        o[1] = u32x4{dw[4], dw[5], dw[6], dw[7]};
    }
}

hipError_t launch_quantize_nv(const uint16_t *src, long long rows, int K, const float *g, uint8_t *codes,
                              uint8_t *scales, uint16_t *dq, hipStream_t st) {
    const long long nb = rows * (K / 16);
    if (nb == 0) return hipSuccess;
    quantize_nv_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, st>>>(src, nb, K, g, codes, scales, dq);
    return hipGetLastError();
}

hipError_t launch_quantize_mx(const uint16_t *src, long long rows, int K, uint8_t *codes, uint8_t *scales,
                              hipStream_t st) {
    const long long nb = rows * (K / 32);
    if (nb == 0) return hipSuccess;
    quantize_mx_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, st>>>(src, nb, K, codes, scales);
    return hipGetLastError();
}

#ifdef MOE_DEBUG
MOE_DEBUG_READER(debug_read_quant)
#endif

}  // namespace moe
