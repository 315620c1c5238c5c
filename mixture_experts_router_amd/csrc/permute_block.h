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
                                           int32_t *__restrict__ inv, [[maybe_unused]] int A) {
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
            *MOE_CHECKED(sorted_ids + pos, 4, sorted_ids, (size_t)A * 4) = a;
            *MOE_CHECKED(inv + a, 4, inv, (size_t)A * 4) = pos;
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
        for (int a0 = 0; a0 < A; a0 += kChunk) rank_chunk(ids, a0, min(A, a0 + kChunk), h, nbits, sorted_ids, inv, A);
}

// Histogram, exclusive scan and stable scatter of A <= 64 assignments
// (ids[a] for a < A, all below 2^NBITS) by a block of E or more threads, from
// the bit planes of the ids: one ballot per bit, taken by every wave (no LDS
// beyond the ids).  For a value v, a walk over the planes from the highest
// bit down keeps the lanes whose ids agree with v on the bits seen so far;
// at each bit set in v, the kept lanes with that bit clear hold smaller ids.
// So the walk gives the number of ids below v (an expert's start) and the
// lanes whose id equals v (its count, and an assignment's stable rank: its
// equals in lower lanes).  Thread i walks expert i; lane a of every wave also
// walks the id of assignment a, and wave 0 stores that rank.  The two walks
// are independent chains without branches, so they run interleaved.
template <int NBITS>
__device__ __forceinline__ void permute_ids_block(const int32_t *ids, int A, int E, int32_t *__restrict__ counts,
                                                  int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_ids,
                                                  int32_t *__restrict__ inv) {
    const int tid = threadIdx.x, lane = tid & 63;
    const bool valid = lane < A;
    const int id = valid ? ids[lane] : 0;
    const uint64_t all = __ballot(valid);
    uint64_t plane[NBITS];
#pragma unroll
    for (int b = 0; b < NBITS; ++b) plane[b] = __ballot(valid && ((id >> b) & 1));
    uint64_t me = all, ma = all;   // lanes agreeing with expert tid / with this lane's id
    int less_e = 0, less_a = 0;
#pragma unroll
    for (int b = NBITS - 1; b >= 0; --b) {
        const uint64_t p = plane[b];
        const bool be = (tid >> b) & 1, ba = (id >> b) & 1;
        less_e += be ? __popcll(me & ~p) : 0;
        less_a += ba ? __popcll(ma & ~p) : 0;
        me &= be ? p : ~p;
        ma &= ba ? p : ~p;
    }
    if (tid < E) {
        counts[tid] = __popcll(me);
        offsets[tid] = less_e;
    }
    if (tid == 0) offsets[E] = A;
    if (tid < 64 && valid) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int pos = less_a + __popcll(ma & below);
        *MOE_CHECKED(sorted_ids + pos, 4, sorted_ids, (size_t)A * 4) = lane;
        *MOE_CHECKED(inv + lane, 4, inv, (size_t)A * 4) = pos;
    }
}

}  // namespace moe
