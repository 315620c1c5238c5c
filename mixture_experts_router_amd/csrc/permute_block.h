// Block-level pieces of the expert permutation, shared by the permutation
// kernels and the fused few-token routing kernel.
#pragma once

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// Mask of the lanes (among those with `valid`) holding the same expert id.
__device__ __forceinline__ uint64_t match_lanes(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const uint64_t ones = __ballot(valid && ((e >> b) & 1));
        m &= ((e >> b) & 1) ? ones : ~ones;
    }
    return m;
}

// Block-wide exclusive scan of E <= 1024 values held one per thread.
__device__ __forceinline__ int block_exclusive_scan(int v, int *sh /* >= blockDim.x ints */) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
        const int add = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    const int incl = sh[tid];
    __syncthreads();
    return incl - v;
}

// Stable rank of the assignments of one chunk (at most kChunk), one wave,
// in 64-lane steps.  cnt[e] holds the next free position of expert e and is
// advanced here.  All expert ids of the chunk are loaded first.
__device__ __forceinline__ void rank_chunk(const int32_t *__restrict__ ids, int a0, int a1,
                                           int *cnt, int nbits, int32_t *__restrict__ sorted_ids,
                                           int32_t *__restrict__ inv) {
    constexpr int kSteps = kChunk / 64;
    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int eid[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int a = a0 + 64 * i + lane;
        eid[i] = a < a1 ? ids[a] : 0;
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int base = a0 + 64 * i;
        if (base >= a1) break;
        const int a = base + lane;
        const bool valid = a < a1;
        const int e = eid[i];
        const uint64_t m = match_lanes(e, valid, nbits);
        const int rank = __popcll(m & below);
        int pos = 0;
        if (valid) pos = cnt[e] + rank;
        // The highest lane of each group advances the counter after every
        // lane of the wave has read it.
        __builtin_amdgcn_wave_barrier();
        if (valid && (m >> lane) == 1ull) cnt[e] = pos + 1;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            sorted_ids[pos] = a;
            inv[a] = pos;
        }
    }
}

// Histogram, exclusive scan and stable scatter of A <= kSmallRouteMaxA
// assignments by one block of 1024 threads.  h (>= E ints, zeroed by the
// caller before this call) and sh (1024 ints) are LDS scratch; ids may live
// in LDS or global memory.
__device__ __forceinline__ void permute_in_block(const int32_t *ids, int A, int E, int nbits, int *h, int *sh,
                                                 int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                 int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv) {
    const int tid = threadIdx.x;
    __syncthreads();
    for (int a = tid; a < A; a += blockDim.x) atomicAdd(&h[ids[a]], 1);
    __syncthreads();
    const int c = tid < E ? h[tid] : 0;
    const int start = block_exclusive_scan(c, sh);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = start;
        h[tid] = start;
    }
    if (tid == 0) offsets[E] = A;
    __syncthreads();
    if (tid < 64)
        for (int a0 = 0; a0 < A; a0 += kChunk) rank_chunk(ids, a0, min(A, a0 + kChunk), h, nbits, sorted_ids, inv);
}

// Histogram, exclusive scan and stable scatter of A <= 64 assignments by one
// wave, lane a holding assignment a.  One pass over the id bits, high to
// low, gives both the number of assignments with a smaller expert id (the
// expert's start) and the mask of lanes with the same id (the stable rank
// within it).  h (>= E ints of LDS, zero on entry) receives the counts.
// Each lane then scans C = ceil(E / 64) <= 16 consecutive experts.
template <int C>
__device__ __forceinline__ void permute_wave(const int32_t *ids, int A, int E, int nbits, int *h,
                                             int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                             int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv) {
    const int lane = threadIdx.x & 63;
    const bool valid = lane < A;
    const int id = valid ? ids[lane] : 0;
    uint64_t m = __ballot(valid);   // valid lanes whose id agrees on the bits seen so far
    int less = 0;
    for (int b = nbits - 1; b >= 0; --b) {
        const bool bit = (id >> b) & 1;
        const uint64_t ones = __ballot(valid && bit);
        if (bit) less += __popcll(m & ~ones);
        m &= bit ? ones : ~ones;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (valid) {
        const int pos = less + __popcll(m & below);
        sorted_ids[pos] = lane;
        inv[lane] = pos;
        if ((m >> lane) == 1ull) h[id] = __popcll(m);   // highest lane of its expert group
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    int c[C];
    int tot = 0;
#pragma unroll
    for (int q = 0; q < C; ++q) {
        const int e = lane * C + q;
        c[q] = e < E ? h[e] : 0;
        tot += c[q];
    }
    int incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    int run = incl - tot;
#pragma unroll
    for (int q = 0; q < C; ++q) {
        const int e = lane * C + q;
        if (e < E) {
            counts[e] = c[q];
            offsets[e] = run;
        }
        run += c[q];
    }
    if (lane == 0) offsets[E] = A;
}

}  // namespace moe
