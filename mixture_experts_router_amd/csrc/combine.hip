// Weighted combine: out[t] = sum_{j<k} w[t, j] * y[inv[t*k + j]], summed in
// fp32 in ascending j and rounded to bf16 once.  This is the local-expert sum
// that the decode path of the pages all-reduces across expert-parallel
// ranks (Gemma-4-26B-A4B optimisation report, section 6.1, MoE row).  Each
// output element is owned by one lane, so there are no atomics and the
// result is bitwise reproducible.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// One wave per (token, 512 consecutive outputs); each lane owns 8
// consecutive outputs (16 bytes).  The token's k rows and weights are
// wave-uniform (scalar loads); the row loads go out in batches of 8.
__global__ __launch_bounds__(64) void combine_kernel(const uint16_t *__restrict__ y,
                                                     const int32_t *__restrict__ inv,
                                                     const float *__restrict__ w,
                                                     uint16_t *__restrict__ out, int H, int k) {
    const int t = blockIdx.x;
    const int c = blockIdx.y * 64 + threadIdx.x;   // 16-byte chunk of the row
    if (c >= H / 8) return;
    const int32_t *ti = inv + (size_t)t * k;
    const float *tw = w + (size_t)t * k;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    // summed in ascending j
    for (int j0 = 0; j0 < k; j0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = min(j0 + u, k - 1);
            v[u] = *reinterpret_cast<const u32x4 *>(y + (size_t)ti[j] * H + c * 8);
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
    *reinterpret_cast<u32x4 *>(out + (size_t)t * H + c * 8) = o;
}

hipError_t launch_combine(const uint16_t *y, const int32_t *inv, const float *w, uint16_t *out, int T,
                          int H, int k, hipStream_t st) {
    if (T == 0) return hipSuccess;
    combine_kernel<<<dim3(T, (H / 8 + 63) / 64), 64, 0, st>>>(y, inv, w, out, H, k);
    return hipGetLastError();
}

}  // namespace moe
