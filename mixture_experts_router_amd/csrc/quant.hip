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
    const u32x4 *p = reinterpret_cast<const u32x4 *>(src + row * K + blk * 32);
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
    *reinterpret_cast<u32x4 *>(codes + row * (K / 2) + blk * 16) = out;
    scales[row * bpr + blk] = (uint8_t)(e + 127);
}

hipError_t launch_quantize_mx(const uint16_t *src, long long rows, int K, uint8_t *codes, uint8_t *scales,
                              hipStream_t st) {
    const long long nb = rows * (K / 32);
    if (nb == 0) return hipSuccess;
    quantize_mx_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, st>>>(src, nb, K, codes, scales);
    return hipGetLastError();
}

}  // namespace moe
