// Router: logits = x W_r^T (+ b) on MFMA, then per token the top-k experts
// and their renormalised softmax weights.
//
// The pages fuse the routing as one gating top-k softmax op (Gemma-4-26B-A4B
// optimisation report, section 5, MoE Router row, 30 calls per step); here
// the router GEMM is a dense contraction on the matrix cores and the top-k is
// k rounds of a wave-wide argmax (one wave per token, the lower expert index
// winning ties), whose softmax weights are taken over the k selected logits.
//
// Logit definition shared by both GEMM paths (split-K below for few tokens,
// the pipelined grouped GEMM engine for many): the K (hidden) axis is cut
// into chunks of 256; each chunk is summed in fp32 by 8 MFMA steps of 32
// products in K order, experts as the A operand (bf16 products are exact in
// fp32), the chunk sums are added in fp64 in chunk order, the bias is added
// in fp64, and the result is rounded to fp32 once.
#include <algorithm>

#include "moe_common.h"
#include "moe_launch.h"
#include "permute_block.h"

namespace moe {

constexpr int kRouteChunk = 256;   // K per fp32 chunk sum (8 MFMA steps)

// ---------------------------------------------------------------- few tokens
// Split-K: one wave owns (16 experts, chunk c, 16 tokens), issues all its
// loads of the chunk at once (the token rows past T are not read) and
// writes the fp32 chunk sums part[c][t][e].
// Many small waves stream the router weight in one memory round trip.
__device__ __forceinline__ void router_partial_wave(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
                                                    float *__restrict__ part, int T, int H, int E, int etile,
                                                    int c, int ttile) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int tok = ttile * 16 + r;   // token row loaded by this lane
    const int e = etile * 16 + r;     // expert row loaded by this lane
    const int k0 = c * kRouteChunk;
    const int nsteps = min(kRouteChunk, H - k0) / 32;
    const uint16_t *arow = x + (size_t)(tok < T ? tok : 0) * H + k0 + 8 * g;
    const uint16_t *brow = wr + (size_t)(e < E ? e : 0) * H + k0 + 8 * g;
    u32x4 a[8], b[8];
    // token columns past T multiply zeros (their sums are never stored), so
    // only real token rows are read
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int su = u < nsteps ? u : 0;
        a[u] = tok < T ? *reinterpret_cast<const u32x4 *>(MOE_CHECKED(arow + 32 * su, 16, x, (size_t)T * H * 2))
                       : u32x4{0u, 0u, 0u, 0u};
        b[u] = *reinterpret_cast<const u32x4 *>(MOE_CHECKED(brow + 32 * su, 16, wr, (size_t)E * H * 2));
    }
    // Experts are the MFMA A operand and tokens the B operand, as in the
    // grouped GEMM engine that computes the router for many tokens: lane
    // (r, g) ends with experts 4g..4g+3 of token r.
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
        if (u < nsteps) acc = mfma16x16x32(b[u], a[u], acc);
    const int t = ttile * 16 + r;
    if (t < T) {
        const int e0 = etile * 16 + 4 * g;
        float *row = part + ((size_t)c * T + t) * E;
        [[maybe_unused]] const size_t ext = (size_t)((H + kRouteChunk - 1) / kRouteChunk) * T * E * 4;
        // one 16-byte store where aligned (a 16-byte aligned buffer and E a
        // multiple of 4, so every row starts at a multiple of 4 floats)
        if (E % 4 == 0 && e0 + 3 < E && (reinterpret_cast<uintptr_t>(part) & 15u) == 0) {
            *reinterpret_cast<f32x4 *>(MOE_CHECKED(row + e0, 16, part, ext)) = acc;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (e0 + q < E) *MOE_CHECKED(row + e0 + q, 4, part, ext) = acc[q];
        }
    }
}

// Block (64 experts, chunk, 16 tokens), one wave per 16 experts.
__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ wr,
                                                             float *__restrict__ part, int T, int H, int E) {
    const int etile = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (etile * 16 >= E) return;
    router_partial_wave(x, wr, part, T, H, E, etile, blockIdx.y, blockIdx.z);
}

// ---------------------------------------------------------------- top-k
// Order-preserving integer key of a float: larger float -> larger key.
// -0.0 is mapped to +0.0 so equal values tie.
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide maximum in every lane: DPP steps inside each row of 16 lanes
// (quad swaps, then the half-row and row mirrors), then the gfx950 lane swaps
// between the two halves and between neighbouring rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // quad [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // quad [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // lanes l and l ^ 32
    v = max(h[0], h[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // rows 0<->1, 2<->3
    return max(r[0], r[1]);
}

// Top-k of one token by one wave; lane l holds experts e = l + 64 i.  Slot j
// takes the largest remaining key, the lowest expert index among equal keys
// (so slots come out ordered by logit descending, index ascending), and the
// weights are exp(l_j - l_0) over their sum, summed in slot order.  If part
// != nullptr the logit is first assembled from nchunks fp32 chunk sums (fp64
// adds in chunk order, plus the fp64 bias, one rounding) and written to
// `logits` if given.  lds_ids (optional): also receives ids[t][slot].
template <int VPL>
__device__ __forceinline__ void topk_token(int t, const float *__restrict__ part, int nchunks,
                                           const float *__restrict__ bias, float *__restrict__ logits,
                                           int32_t *__restrict__ ids, float *__restrict__ wts, int T, int E,
                                           int k, int32_t *lds_ids) {
    const int lane = threadIdx.x & 63;
    uint32_t key[VPL];   // 0 = no expert (past E) or already taken
    if (part) {
        // Values in groups of IB; all chunk-sum loads of a batch (every chunk
        // for H <= 4096 and E <= 128) are issued before the first add.
        constexpr int IB = VPL < 4 ? VPL : 4;
        constexpr int CB = IB <= 2 ? 16 : 4;
#pragma unroll
        for (int i0 = 0; i0 < VPL; i0 += IB) {
            double s[IB];
            float b[IB];
#pragma unroll
            for (int i = 0; i < IB; ++i) {
                const int e = lane + 64 * (i0 + i);
                b[i] = (bias && e < E) ? bias[e] : 0.f;
                s[i] = 0.0;
            }
            for (int c0 = 0; c0 < nchunks; c0 += CB) {
                float pv[IB][CB];
#pragma unroll
                for (int i = 0; i < IB; ++i) {
                    const int e = min(lane + 64 * (i0 + i), E - 1);
#pragma unroll
                    for (int u = 0; u < CB; ++u)
                        pv[i][u] = *MOE_CHECKED(part + ((size_t)min(c0 + u, nchunks - 1) * T + t) * E + e, 4, part,
                                                (size_t)nchunks * T * E * 4);
                }
#pragma unroll
                for (int i = 0; i < IB; ++i)
#pragma unroll
                    for (int u = 0; u < CB; ++u)
                        if (c0 + u < nchunks) s[i] += (double)pv[i][u];
            }
#pragma unroll
            for (int i = 0; i < IB; ++i) {
                const int e = lane + 64 * (i0 + i);
                key[i0 + i] = 0u;
                if (e < E) {
                    const float v = (float)(s[i] + (double)b[i]);
                    if (logits) *MOE_CHECKED(logits + (size_t)t * E + e, 4, logits, (size_t)T * E * 4) = v;
                    key[i0 + i] = order_key(v);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + 64 * i;
            key[i] = e < E ? order_key(*MOE_CHECKED(logits + (size_t)t * E + e, 4, logits, (size_t)T * E * 4)) : 0u;
        }
    }
    // k rounds of wave argmax; lane j keeps slot j.
    int my_idx = 0;
    uint32_t my_key = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t lm = key[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i) lm = max(lm, key[i]);
        const uint32_t km = wave_max_u32(lm);
        // the lowest expert index holding km: the lowest lane of the lowest
        // i with a hit (scalar selects, no branch per i)
        int sel = 0;
#pragma unroll
        for (int i = VPL - 1; i >= 0; --i) {
            const uint64_t hit = __ballot(key[i] == km);
            // (bit 63 keeps the count defined for an empty mask, whose
            // result is not selected, and changes no nonzero one)
            sel = hit ? 64 * i + (int)__builtin_ctzll(hit | (1ull << 63)) : sel;
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (64 * i + lane == sel) key[i] = 0u;
        if (lane == j) {
            my_idx = sel;
            my_key = km;
        }
    }
    // weights: exp(l_j - l_0) in every slot lane at once, their sum in slot order
    const float top = key_value((uint32_t)__builtin_amdgcn_readfirstlane((int)my_key));
    const float ex = lane < k ? expf(key_value(my_key) - top) : 0.f;
    float sum = 0.f;
    for (int m = 0; m < k; ++m) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), m));
    if (lane < k) {
        *MOE_CHECKED(ids + (size_t)t * k + lane, 4, ids, (size_t)T * k * 4) = my_idx;
        *MOE_CHECKED(wts + (size_t)t * k + lane, 4, wts, (size_t)T * k * 4) = ex / sum;
        if (lds_ids) lds_ids[t * k + lane] = my_idx;
    }
}

// One wave per token, four tokens per workgroup.
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ part, int nchunks,
                                                   const float *__restrict__ bias, float *__restrict__ logits,
                                                   int32_t *__restrict__ ids, float *__restrict__ wts, int T,
                                                   int E, int k) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_token<VPL>(t, part, nchunks, bias, logits, ids, wts, T, E, k, nullptr);
}

// Few tokens, one workgroup of 16 waves: the top-k of every token, then the
// expert histogram, its scan and the stable scatter of the assignments, all
// from the routing table kept in LDS (it never makes a round trip through
// global memory before the scatter).  Up to 64 assignments the permutation
// comes from the ballots of the ids' bit planes, one expert per thread.
template <int VPL>
__device__ __forceinline__ void topk_permute_block(const float *__restrict__ part, int nchunks,
                                                   const float *__restrict__ bias, float *__restrict__ logits,
                                                   int32_t *__restrict__ ids, float *__restrict__ wts,
                                                   int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv,
                                                   int T, int E, int k, int nbits, int32_t *s_ids, int *h, int *sh) {
    const int tid = threadIdx.x, wave = tid >> 6;
    const int A = T * k;
    if (tid < E) h[tid] = 0;
    for (int t = wave; t < T; t += 16) topk_token<VPL>(t, part, nchunks, bias, logits, ids, wts, T, E, k, s_ids);
    __syncthreads();
    if (A <= 64) {
        // ids below 64 VPL = 2^(6 + log2 VPL)
        constexpr int NBITS = 6 + (VPL >= 2) + (VPL >= 4) + (VPL >= 8) + (VPL >= 16);
        permute_ids_block<NBITS>(s_ids, A, E, counts, offsets, sorted_ids, inv);
    } else {
        permute_in_block(s_ids, A, E, nbits, h, sh, counts, offsets, sorted_ids, inv);
    }
}

// The whole few-token routing in one launch.  Every block first computes
// its share of the router chunk sums (work item = 16 experts of one chunk
// and 16 tokens, one wave each, the first `wpb` waves of a block busy: few
// items per block spread the router weight's bytes over many CUs, whose load
// path they would otherwise queue on); the last block to finish -- found
// with a completion counter -- then runs the top-k and the permutation over
// all of them.
// Release/acquire: each block's sums are made visible device-wide (agent-
// scope fence) before its counter increment, and the last block fences
// again before reading them.  The counter wraps back to zero on the last
// increment, so it is zero again for the next call.
template <int VPL>
__global__ __launch_bounds__(1024) void route_permute_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, float *__restrict__ part, int H,
    uint32_t *__restrict__ done, const float *__restrict__ bias, float *__restrict__ logits,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv, int T, int E,
    int k, int nbits, int nchunks, int wpb) {
    __shared__ int32_t s_ids[kSmallRouteMaxA];
    __shared__ int h[1024];
    __shared__ int sh[1024];
    __shared__ int s_last;
    const int wave = threadIdx.x >> 6, netiles = (E + 15) / 16;
    const int item = blockIdx.x * wpb + wave;   // (etile, chunk, token tile), etile fastest
    if (wave < wpb && item < netiles * nchunks * ((T + 15) / 16))
        router_partial_wave(x, wr, part, T, H, E, item % netiles, (item / netiles) % nchunks,
                            item / (netiles * nchunks));
    // Every wave waits until its stores are complete in this XCD's L2; after
    // the barrier one thread makes them visible device-wide (L2 write-back),
    // counts the block done and, in the last block, invalidates the caches
    // before any wave reads the other blocks' sums.  (Fencing in every wave
    // would cost one L2 write-back per wave.)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t nblocks = gridDim.x;
        __threadfence();
        const bool last = atomicInc(done, nblocks - 1) == nblocks - 1;
        if (last) __threadfence();
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    topk_permute_block<VPL>(part, nchunks, bias, logits, ids, wts, counts, offsets, sorted_ids, inv, T, E, k,
                            nbits, s_ids, h, sh);
}

// ---------------------------------------------------------------- launchers
int router_chunks(int H) { return (H + kRouteChunk - 1) / kRouteChunk; }

bool router_uses_partials(int T) { return T <= kRouterSplitMaxT; }

hipError_t launch_router_partials(const uint16_t *x, const uint16_t *wr, float *part, int T, int H, int E,
                                  hipStream_t st) {
    dim3 grid((E + 63) / 64, router_chunks(H), (T + 15) / 16);
    router_partial_kernel<<<grid, 256, 0, st>>>(x, wr, part, T, H, E);
    return hipGetLastError();
}

// The last block runs the top-k of every token, one per wave: beyond its 16
// waves a wave would take tokens one after another, and the staged launches
// (chunk sums, a top-k launch with a wave per token, the permutation) are
// faster (measured, layer step at 24 / 32 / 64 tokens: 225.3 / 244.4 /
// 275.6 us single-launch against 222.3 / 238.9 / 259.8 us staged).
bool route_permute_fits(int T, int k) {
    return T <= kFusedRouteMaxT && router_uses_partials(T) && T * k <= kSmallRouteMaxA;
}

hipError_t launch_route_permute(const uint16_t *x, const uint16_t *wr, float *part, uint32_t *done,
                                const float *bias, float *logits, int32_t *ids, float *w, int32_t *counts,
                                int32_t *offsets, int32_t *sorted_ids, int32_t *inv, int T, int H, int E, int k,
                                hipStream_t st) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int vpl = (E + 63) / 64;
    // Work items of 16 experts x one chunk x 16 tokens, two per block (up to
    // 512 blocks; more items share blocks).  Measured on the decode shape
    // (8 tokens, 128 experts, hidden 2816: 88 items), 11 blocks of eight busy
    // waves -> 44 blocks of two: the launch 9.9 -> 8.5 us back to back, the
    // layer step 100.4 -> 98.6 us (with the bit-plane permutation).
    const int nchunks = router_chunks(H);
    const int items = ((E + 15) / 16) * nchunks * ((T + 15) / 16);
    const int wpb = std::min(16, std::max(2, (items + 511) / 512));
    const int blocks = (items + wpb - 1) / wpb;
#define MOE_ROUTE_PERM(V)                                                                                          \
    route_permute_kernel<V><<<blocks, 1024, 0, st>>>(x, wr, part, H, done, bias, logits, ids, w, counts, offsets, \
                                                     sorted_ids, inv, T, E, k, nbits, nchunks, wpb)
    if (vpl <= 1) MOE_ROUTE_PERM(1);
    else if (vpl <= 2) MOE_ROUTE_PERM(2);
    else if (vpl <= 4) MOE_ROUTE_PERM(4);
    else if (vpl <= 8) MOE_ROUTE_PERM(8);
    else MOE_ROUTE_PERM(16);
#undef MOE_ROUTE_PERM
    return hipGetLastError();
}

hipError_t launch_topk(const float *part, int nchunks, const float *bias, float *logits, int32_t *ids,
                       float *w, int T, int E, int k, hipStream_t st) {
    dim3 grid((T + 3) / 4);
    const int vpl = (E + 63) / 64;
#define MOE_TOPK(V) topk_kernel<V><<<grid, 256, 0, st>>>(part, nchunks, bias, logits, ids, w, T, E, k)
    if (vpl <= 1) MOE_TOPK(1);
    else if (vpl <= 2) MOE_TOPK(2);
    else if (vpl <= 4) MOE_TOPK(4);
    else if (vpl <= 8) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

#ifdef MOE_DEBUG
MOE_DEBUG_READER(debug_read_route)
#endif

}  // namespace moe
