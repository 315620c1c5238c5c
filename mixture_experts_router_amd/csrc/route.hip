// Router: logits = x W_r^T (+ b) on MFMA, then per token the top-k experts
// and their renormalised softmax weights, one wavefront per token.
//
// The pages fuse the routing as one gating top-k softmax op (Gemma-4-26B-A4B
// optimisation report, section 5, MoE Router row, 30 calls per step); here
// the router GEMM is a dense contraction on the matrix cores and the top-k is
// a wave-wide lexicographic argmax repeated k times.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// ---------------------------------------------------------------- router GEMM
// Each wave owns SM x SN tiles of 16x16 (tokens x experts); the workgroup has
// WM x WN x WK waves: WM along tokens, WN along experts and WK splitting the
// K (hidden) steps round-robin.  Products of bf16 are exact in fp32; each
// wave sums blocks of up to 8 MFMA steps (256 products) in fp32 and adds the
// block sums into fp64, and the WK partials are added in fixed order, so the
// logit is rounded to fp32 once and the result does not depend on timing.
template <int SM, int SN, int WM, int WN, int WK>
__global__ __launch_bounds__(256) void router_gemm_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int H, int E) {
    static_assert(WM * WN * WK == 4, "four waves");
    constexpr int TM = 16 * SM * WM;   // tokens per workgroup
    constexpr int TN = 16 * SN * WN;   // experts per workgroup
    constexpr int kRed = (WK > 1 ? (WK - 1) * WM * WN : 1) * SM * SN * 4 * 64;
    __shared__ double red[kRed];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wk = wave % WK, wn = (wave / WK) % WN, wm = wave / (WK * WN);
    const int r = lane & 15, g = lane >> 4;
    const int tok0 = blockIdx.x * TM + wm * 16 * SM;
    const int exp0 = blockIdx.y * TN + wn * 16 * SN;

    const uint16_t *arow[SM];
    bool aok[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        int t = tok0 + 16 * i + r;
        aok[i] = t < T;
        arow[i] = x + (size_t)(aok[i] ? t : 0) * H + 8 * g;
    }
    const uint16_t *brow[SN];
    bool bok[SN];
#pragma unroll
    for (int j = 0; j < SN; ++j) {
        int e = exp0 + 16 * j + r;
        bok[j] = e < E;
        brow[j] = wr + (size_t)(bok[j] ? e : 0) * H + 8 * g;
    }

    double acc64[SM][SN][4];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc64[i][j][q] = 0.0;

    const int nsteps = H / 32;
    for (int s0 = wk; s0 < nsteps; s0 += 8 * WK) {
        f32x4 acc[SM][SN];
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = s0 + u * WK;
            if (s < nsteps) {
                u32x4 a[SM], b[SN];
#pragma unroll
                for (int i = 0; i < SM; ++i)
                    a[i] = aok[i] ? *reinterpret_cast<const u32x4 *>(arow[i] + 32 * s) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    b[j] = bok[j] ? *reinterpret_cast<const u32x4 *>(brow[j] + 32 * s) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
            }
        }
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc64[i][j][q] += (double)acc[i][j][q];
    }

    // Fixed-order reduction of the WK partials through LDS.
    if constexpr (WK > 1) {
        const int slot = wm * WN + wn;
        if (wk > 0) {
            double *dst = red + ((wk - 1) * WM * WN + slot) * SM * SN * 256;
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        dst[((i * SN + j) * 4 + q) * 64 + lane] = acc64[i][j][q];
        }
        __syncthreads();
        if (wk != 0) return;
#pragma unroll
        for (int w = 1; w < WK; ++w) {
            const double *src = red + ((w - 1) * WM * WN + slot) * SM * SN * 256;
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc64[i][j][q] += src[((i * SN + j) * 4 + q) * 64 + lane];
        }
    }

#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            const int e = exp0 + 16 * j + r;
            if (e >= E) continue;
            const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = tok0 + 16 * i + 4 * g + q;
                if (t < T) logits[(size_t)t * E + e] = (float)(acc64[i][j][q] + b);
            }
        }
}

// ---------------------------------------------------------------- top-k
// One wave per token.  Lane l holds logits e = l + 64 i.  Each of the k rounds
// takes the lexicographic maximum of (logit, -index) over the wave and retires
// it, so ties resolve to the lower expert index and slots come out in
// (logit descending, index ascending) order.  Weights: exp(l_j - l_0) divided
// by their sum over the k slots.
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wts, int T, int E, int k) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *L = logits + (size_t)t * E;
    float v[VPL];
    bool live[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        v[i] = live[i] ? L[e] : 0.f;
    }
    float my_v = 0.f;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
        float bv = 0.f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (live[i] && (bi < 0 || v[i] > bv)) { bv = v[i]; bi = lane + 64 * i; }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
        }
        if ((bi & 63) == lane) {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (i == (bi >> 6)) live[i] = false;
        }
        if (lane == j) { my_v = bv; my_i = bi; }
    }
    const float m = __shfl(my_v, 0, 64);
    float ex = lane < k ? expf(my_v - m) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_i;
        wts[(size_t)t * k + lane] = ex / sum;
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_router_gemm(const uint16_t *x, const uint16_t *wr, const float *bias,
                              float *logits, int T, int H, int E, hipStream_t st) {
    if (T <= 256) {
        // Few tokens: 16x16 tiles with the hidden dimension split over the
        // four waves, so the router weight is streamed by E/16 workgroups.
        dim3 grid((T + 15) / 16, (E + 15) / 16);
        router_gemm_kernel<1, 1, 1, 1, 4><<<grid, 256, 0, st>>>(x, wr, bias, logits, T, H, E);
    } else {
        dim3 grid((T + 63) / 64, (E + 31) / 32);
        router_gemm_kernel<2, 1, 2, 2, 1><<<grid, 256, 0, st>>>(x, wr, bias, logits, T, H, E);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int32_t *ids, float *w, int T, int E, int k,
                       hipStream_t st) {
    dim3 grid((T + 3) / 4);
    const int vpl = (E + 63) / 64;
    if (vpl <= 1) topk_kernel<1><<<grid, 256, 0, st>>>(logits, ids, w, T, E, k);
    else if (vpl <= 2) topk_kernel<2><<<grid, 256, 0, st>>>(logits, ids, w, T, E, k);
    else if (vpl <= 4) topk_kernel<4><<<grid, 256, 0, st>>>(logits, ids, w, T, E, k);
    else if (vpl <= 8) topk_kernel<8><<<grid, 256, 0, st>>>(logits, ids, w, T, E, k);
    else topk_kernel<16><<<grid, 256, 0, st>>>(logits, ids, w, T, E, k);
    return hipGetLastError();
}

}  // namespace moe
