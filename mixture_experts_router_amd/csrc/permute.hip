// Dispatch bookkeeping: per-expert counts, their prefix sum and the stable
// expert-grouped order of the (token, slot) assignments.  These counts are
// the data-dependent split sizes of the dispatch (Gemma-4-26B-A4B
// optimisation report, section 6.1, MoE row).
//
// Deterministic and free of global atomics: each block of kChunk assignments
// builds its histogram in LDS, one block scans the block histograms, and each
// block then ranks its assignments in order (wave ballots give the rank
// among equal experts inside 64 lanes; per-wave counts, scanned per expert
// over the block's waves, carry it across the block).
#include "moe_common.h"
#include "moe_launch.h"
#include "permute_block.h"

namespace moe {

// Block b counts experts of assignments [b*kChunk, (b+1)*kChunk).
__global__ __launch_bounds__(256) void hist_kernel(const int32_t *__restrict__ ids,
                                                   int32_t *__restrict__ block_hist, int A, int E) {
    extern __shared__ int32_t h[];
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int a0 = blockIdx.x * kChunk;
    const int a1 = min(A, a0 + kChunk);
    for (int a = a0 + threadIdx.x; a < a1; a += blockDim.x) atomicAdd(&h[ids[a]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) block_hist[(size_t)blockIdx.x * E + e] = h[e];
}

// One block of 1024 threads: counts[e] = sum over blocks; offsets = exclusive
// scan; block_hist[b][e] is replaced by the absolute start of block b's
// assignments of expert e.
// The block histograms are read in batches of 16 before any is rewritten, so
// the loads of a batch are in flight together.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *__restrict__ block_hist,
                                                    int32_t *__restrict__ counts,
                                                    int32_t *__restrict__ offsets, int NB, int E, int A) {
    __shared__ int sh[1024];
    const int e = threadIdx.x;
    int total = 0;
    if (e < E)
        for (int b0 = 0; b0 < NB; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = (b0 + i < NB) ? block_hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int cnt = c[i];
                c[i] = total;      // exclusive start within the expert
                total += cnt;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (b0 + i < NB) block_hist[(size_t)(b0 + i) * E + e] = c[i];
        }
    const int start = block_exclusive_scan(e < E ? total : 0, sh);
    if (e < E) {
        counts[e] = total;
        offsets[e] = start;
        for (int b0 = 0; b0 < NB; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = (b0 + i < NB) ? block_hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (b0 + i < NB) block_hist[(size_t)(b0 + i) * E + e] = c[i] + start;
        }
    }
    if (e == 0) offsets[E] = A;
}

// Positions for one chunk of kChunk assignments, one per thread (16 waves):
// each wave ranks its 64 assignments among equal experts (ballots) and
// records its count of each expert (at most 64: one byte); a lane's position
// is then the block's base for its expert, plus the counts of that expert in
// the earlier waves, plus its rank.  base: LDS, [E]; wc: LDS, [16][E].
constexpr int kScatterWaves = kChunk / 64;
__device__ __forceinline__ void scatter_chunk(const int32_t *__restrict__ ids, const int *base, uint8_t *wc,
                                              int32_t *__restrict__ sorted_ids, int32_t *__restrict__ inv, int A,
                                              int E, int nbits) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int a = blockIdx.x * kChunk + tid;
    const bool valid = a < A;
    const int e = valid ? ids[a] : 0;
    const uint64_t m = match_lanes(e, valid, nbits);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (valid && (m >> lane) == 1ull) wc[wave * E + e] = (uint8_t)__popcll(m);   // highest lane of its group
    __syncthreads();
    if (valid) {
        int pos = base[e] + __popcll(m & below);
        for (int w = 0; w < wave; ++w) pos += wc[w * E + e];
        *MOE_CHECKED(sorted_ids + pos, 4, sorted_ids, (size_t)A * 4) = a;
        *MOE_CHECKED(inv + a, 4, inv, (size_t)A * 4) = pos;
    }
}

// The scatter after scan_kernel: block_base[b][e] is chunk b's start of
// expert e.
__global__ __launch_bounds__(kChunk) void scatter_kernel(const int32_t *__restrict__ ids,
                                                         const int32_t *__restrict__ block_base,
                                                         int32_t *__restrict__ sorted_ids,
                                                         int32_t *__restrict__ inv, int A, int E, int nbits) {
    extern __shared__ int dyn[];
    int *base = dyn;                                          // [E]
    uint8_t *wc = reinterpret_cast<uint8_t *>(dyn + E);       // [16][E]
    for (int i = threadIdx.x; i < kScatterWaves * E; i += kChunk) wc[i] = 0;
    for (int x = threadIdx.x; x < E; x += kChunk) base[x] = block_base[(size_t)blockIdx.x * E + x];
    __syncthreads();
    scatter_chunk(ids, base, wc, sorted_ids, inv, A, E, nbits);
}

// Scan and scatter in one launch for at most kScanFuseMaxBlocks chunks: every
// block sums the chunk histograms per expert itself (chunks before its own
// give its bases, all chunks the expert totals), scans the totals over the
// experts, and block 0 writes counts and offsets.  E <= kChunk: one thread
// per expert.
constexpr int kScanFuseMaxBlocks = 64;
__global__ __launch_bounds__(kChunk) void scan_scatter_kernel(const int32_t *__restrict__ ids,
                                                              const int32_t *__restrict__ block_hist,
                                                              int32_t *__restrict__ counts,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ sorted_ids,
                                                              int32_t *__restrict__ inv, int A, int E, int nbits,
                                                              int NB) {
    extern __shared__ int dyn[];
    __shared__ int sh[kChunk];
    int *base = dyn;                                          // [E]
    uint8_t *wc = reinterpret_cast<uint8_t *>(dyn + E);       // [16][E]
    const int x = threadIdx.x;
    for (int i = x; i < kScatterWaves * E; i += kChunk) wc[i] = 0;
    int tot = 0, pre = 0;
    if (x < E) {
        // all chunk counts of the expert in flight at once (NB <= 64)
        int c[kScanFuseMaxBlocks];
#pragma unroll
        for (int b = 0; b < kScanFuseMaxBlocks; ++b) c[b] = b < NB ? block_hist[(size_t)b * E + x] : 0;
#pragma unroll
        for (int b = 0; b < kScanFuseMaxBlocks; ++b) {
            pre += b < (int)blockIdx.x ? c[b] : 0;
            tot += c[b];
        }
    }
    const int start = block_exclusive_scan(tot, sh);
    if (x < E) {
        base[x] = start + pre;
        if (blockIdx.x == 0) {
            counts[x] = tot;
            offsets[x] = start;
        }
    }
    if (blockIdx.x == 0 && x == 0) offsets[E] = A;
    __syncthreads();
    scatter_chunk(ids, base, wc, sorted_ids, inv, A, E, nbits);
}

// Everything in one block of 1024 threads when A <= kChunk: histogram,
// scan, scatter.
__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t *__restrict__ ids,
                                                             int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ sorted_ids,
                                                             int32_t *__restrict__ inv, int A, int E, int nbits) {
    __shared__ int h[1024];
    __shared__ int sh[1024];
    if ((int)threadIdx.x < E) h[threadIdx.x] = 0;
    permute_in_block(ids, A, E, nbits, h, sh, counts, offsets, sorted_ids, inv);
}

// x_perm[p] = x[sorted_ids[p] / k]: one wave per row, 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ sorted_ids,
                                                          uint16_t *__restrict__ x_perm, int A, int H, int k) {
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= A) return;
    const int lane = threadIdx.x & 63;
    const int t = sorted_ids[p] / k;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)t * H);
    u32x4 *dst = reinterpret_cast<u32x4 *>(x_perm + (size_t)p * H);
    for (int c = lane; c < H / 8; c += 64)
        *MOE_CHECKED(dst + c, 16, x_perm, (size_t)A * H * 2) = *MOE_CHECKED(src + c, 16, x, (size_t)A / k * H * 2);
}

static int bits_for(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

hipError_t launch_permute(const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_ids, int32_t *inv, int32_t *block_hist, int A, int E,
                          hipStream_t st) {
    const int nbits = bits_for(E);
    if (A <= kChunk) {
        permute_small_kernel<<<1, 1024, 0, st>>>(ids, counts, offsets, sorted_ids, inv, A, E, nbits);
        return hipGetLastError();
    }
    const int NB = (A + kChunk - 1) / kChunk;
    const size_t lds = E * sizeof(int32_t) + kScatterWaves * E;
    hist_kernel<<<NB, 256, E * sizeof(int32_t), st>>>(ids, block_hist, A, E);
    if (NB <= kScanFuseMaxBlocks) {
        scan_scatter_kernel<<<NB, kChunk, lds, st>>>(ids, block_hist, counts, offsets, sorted_ids, inv, A, E, nbits,
                                                     NB);
        return hipGetLastError();
    }
    scan_kernel<<<1, 1024, 0, st>>>(block_hist, counts, offsets, NB, E, A);
    scatter_kernel<<<NB, kChunk, lds, st>>>(ids, block_hist, sorted_ids, inv, A, E, nbits);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t *x, const int32_t *sorted_ids, uint16_t *x_perm,
                              int A, int H, int k, hipStream_t st) {
    gather_rows_kernel<<<(A + 3) / 4, 256, 0, st>>>(x, sorted_ids, x_perm, A, H, k);
    return hipGetLastError();
}

#ifdef MOE_DEBUG
MOE_DEBUG_READER(debug_read_permute)
#endif

}  // namespace moe
