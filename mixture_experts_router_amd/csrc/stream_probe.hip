// Load-only streaming probes: how fast HBM delivers bytes through the same
// direct-to-LDS loads the grouped GEMMs use, for a plain stream and for the
// launch shapes of the decode GEMMs, with no arithmetic at all.  They are
// the reference the GEMMs' achieved bandwidth is read against (what the
// chip streams at that launch shape).  One more probe reads LDS alone, for
// the LDS read rate the large GEMM tiles' fragment loads are bounded by.
// `bench.py --stream-probe` times them.  Built into libmoe_probe.so of its
// own: the layer never calls it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_probe.h"

namespace {

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16-byte direct global->LDS load of one wave (lane l's 16 bytes land at
// lds + 16 l), with the streaming hint: every probe byte is read once.
__device__ __forceinline__ void dma16(const void *g, const void *lds) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(l) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(VM), other counters left at their maxima.
template <int VM>
__device__ __forceinline__ void wait_vm() {
    static_assert(VM >= 0 && VM < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Plain stream: workgroup w (4 waves) reads PER_WG consecutive bytes from
// w * PER_WG, 1 KB per wave and load, DEPTH loads in flight per wave.
template <size_t PER_WG, int DEPTH>
__global__ __launch_bounds__(256) void linear_kernel(const uint8_t *buf, int *sink) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * DEPTH * 1024];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint8_t *base = buf + (size_t)blockIdx.x * PER_WG;
    constexpr int N = (int)(PER_WG / 4096);   // 4 KB per workgroup and step
    for (int i = 0; i < N; ++i) {
        dma16(base + (size_t)i * 4096 + wave * 1024 + lane * 16, ring + ((i % DEPTH) * 4 + wave) * 1024);
        if (i + 1 >= DEPTH) wait_vm<DEPTH - 1>();
    }
    wait_vm<0>();
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = ring[lane];
}

// GEMM-shaped stream: workgroup w reads ROWS rows of RL bytes starting at
// row w * ROWS into a two-stage LDS ring, SB bytes per step, with a wait and
// a barrier per step like the GEMM's K loop.  PIECE > 0: a step reads SB /
// PIECE rows x PIECE bytes (row groups outer, column pieces inner, as the K
// loop reads a weight tile); PIECE == 0: SB consecutive bytes.
template <int RL, int ROWS, int SB, int PIECE>
__device__ __forceinline__ void rows_stream(const uint8_t *base, uint8_t *ring, int &s) {
    constexpr int PER_WAVE = SB / 4096;
    constexpr int STEPS = ROWS * RL / SB;
    static_assert(SB % 4096 == 0 && (ROWS * RL) % SB == 0, "whole steps");
    static_assert(PIECE == 0 || (SB % PIECE == 0 && RL % PIECE == 0 && PIECE % 16 == 0 && ROWS % (SB / PIECE) == 0),
                  "whole pieces");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int st = 0; st < STEPS; ++st, ++s) {
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int flat = (q * 4 + wave) * 1024 + lane * 16;   // byte within the step's block
            size_t off;
            if (PIECE == 0) {
                off = (size_t)st * SB + flat;
            } else {
                constexpr int R = PIECE ? SB / PIECE : 1, CSTEPS = PIECE ? RL / PIECE : 1;
                const int rg = st / CSTEPS, cs = st % CSTEPS;
                off = (size_t)(rg * R + flat / PIECE) * RL + cs * PIECE + flat % PIECE;
            }
            dma16(base + off, ring + (s % 2) * SB + (q * 4 + wave) * 1024);
        }
        if (st + 1 >= 2 || s >= 1) wait_vm<PER_WAVE>();
        __syncthreads();
    }
    wait_vm<0>();
    __syncthreads();
}

// The same byte stream in the grouped GEMM's two-stage order: a step's
// loads are issued after the barrier that publishes the previous step (whose
// buffer they overwrite was consumed before it), so one step is in flight
// while a wave waits, where rows_stream keeps two.
template <int RL, int ROWS, int SB, int PIECE>
__global__ __launch_bounds__(256) void rows_gemm_order_kernel(const uint8_t *buf, int *sink) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * SB];
    constexpr int PER_WAVE = SB / 4096;
    constexpr int STEPS = ROWS * RL / SB;
    static_assert(SB % 4096 == 0 && (ROWS * RL) % SB == 0 && SB % PIECE == 0 && RL % PIECE == 0 &&
                  PIECE % 16 == 0 && ROWS % (SB / PIECE) == 0, "whole steps and pieces");
    constexpr int R = SB / PIECE, CSTEPS = RL / PIECE;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint8_t *base = buf + (size_t)blockIdx.x * ROWS * RL;
    auto issue = [&](int st) {
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int flat = (q * 4 + wave) * 1024 + lane * 16;
            const int rg = st / CSTEPS, cs = st % CSTEPS;
            dma16(base + (size_t)(rg * R + flat / PIECE) * RL + cs * PIECE + flat % PIECE,
                  ring + (st % 2) * SB + (q * 4 + wave) * 1024);
        }
    };
    issue(0);
    for (int st = 0; st < STEPS; ++st) {
        wait_vm<0>();
        __syncthreads();
        if (st + 1 < STEPS) issue(st + 1);
    }
    wait_vm<0>();
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = ring[lane];
}

template <int RL, int ROWS, int SB, int PIECE>
__global__ __launch_bounds__(256) void rows_kernel(const uint8_t *buf, int *sink) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * SB];
    int s = 0;
    rows_stream<RL, ROWS, SB, PIECE>(buf + (size_t)blockIdx.x * ROWS * RL, ring, s);
    if (threadIdx.x == 0) sink[blockIdx.x] = ring[threadIdx.x & 63];
}

// Both decode GEMMs' bytes in one launch: workgroup w = 11 e + n reads the
// 128 gate/up rows (5632 bytes each) of column tile n of expert e, then the
// 128-byte column slice n of that expert's 2816 down rows (1408 bytes each).
constexpr int kExperts = 45, kTiles = 11;
constexpr size_t kGuBytes = (size_t)kExperts * 1408 * 5632, kDnBytes = (size_t)kExperts * 2816 * 1408;
__global__ __launch_bounds__(256) void fused_kernel(const uint8_t *buf, int *sink) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * 32768];
    const int e = blockIdx.x / kTiles, n = blockIdx.x % kTiles;
    int s = 0;
    rows_stream<5632, 128, 32768, 256>(buf + ((size_t)e * 1408 + n * 128) * 5632, ring, s);
    // the down slice: 22 steps of 128 rows x 128 bytes at a 1408-byte stride
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint8_t *dn = buf + kGuBytes + (size_t)e * 2816 * 1408 + n * 128;
    for (int c = 0; c < 22; ++c, ++s) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int flat = (q * 4 + wave) * 1024 + lane * 16;
            dma16(dn + (size_t)(c * 128 + flat / 128) * 1408 + flat % 128, ring + (s % 4) * 16384 + (q * 4 + wave) * 1024);
        }
        if (c >= 3) wait_vm<12>();
        __syncthreads();
    }
    wait_vm<0>();
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = ring[lane];
}

// LDS read rate: 256 workgroups of 1024 threads (16 waves, one workgroup per
// CU), each thread reading 16 bytes per ds_read_b128 from a 64 KB LDS buffer
// at consecutive 16-byte addresses across a wave (no bank conflicts).
constexpr int kLdsIters = 1000;
__global__ __launch_bounds__(1024) void lds_kernel(int *sink) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) unsigned buf[16384];
    for (int i = threadIdx.x; i < 16384; i += 1024) buf[i] = i * 2654435761u;
    __syncthreads();
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int base = (threadIdx.x * 4) & 16383;
    for (int it = 0; it < kLdsIters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int idx = (base + u * 1024 + it * 4) & 16380;   // 16-byte aligned, inside the buffer
            acc ^= *reinterpret_cast<const u32x4 *>(&buf[idx]);
        }
    }
    // a condition on every thread's sum keeps every read
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x12345678u) sink[blockIdx.x] = (int)acc[0];
}

struct Probe {
    const char *name;
    size_t bytes;       // read by one launch (from LDS for the LDS probe)
    size_t footprint;   // needed in the buffer
    int wgs;
};
constexpr size_t kStream = (size_t)1024 << 21, kGu = (size_t)495 * 128 * 5632, kDn = (size_t)990 * 128 * 1408;
constexpr Probe kProbes[] = {
    {"stream: 1024 workgroups x 2 MiB, consecutive, 8 KB in flight per wave", kStream, kStream, 1024},
    {"decode gate/up shape: 495 x 128 rows x 5632 B, steps of 128 rows x 256 B", kGu, kGu, 495},
    {"decode gate/up shape: 495 x 720 KB, steps of 32 KB consecutive", kGu, kGu, 495},
    {"decode gate/up shape, the GEMM's order (one step in flight)", kGu, kGu, 495},
    {"decode down shape: 990 x 128 rows x 1408 B, steps of 128 rows x 128 B", kDn, kDn, 990},
    {"decode down shape: 990 x 176 KB, steps of 16 KB consecutive", kDn, kDn, 990},
    {"decode down shape, the GEMM's order (one step in flight)", kDn, kDn, 990},
    {"both decode GEMMs in one launch: 495 x (720 KB gate/up rows + 360 KB down slice)", kGuBytes + kDnBytes,
     kGuBytes + kDnBytes, 495},
    {"LDS read: 256 workgroups x 16 waves, ds_read_b128, consecutive 16 B per lane",
     (size_t)256 * 1024 * 16 * 16 * kLdsIters, 0, 256},
};
constexpr int kNumProbes = (int)(sizeof(kProbes) / sizeof(kProbes[0]));

}  // namespace

extern "C" {

int moe_probe_count(void) { return kNumProbes; }
const char *moe_probe_name(int kind) { return kind >= 0 && kind < kNumProbes ? kProbes[kind].name : nullptr; }
size_t moe_probe_bytes(int kind) { return kind >= 0 && kind < kNumProbes ? kProbes[kind].bytes : 0; }
size_t moe_probe_footprint(int kind) { return kind >= 0 && kind < kNumProbes ? kProbes[kind].footprint : 0; }

int moe_probe_launch(int kind, const void *buf, size_t buf_bytes, int *sink, void *stream) {
    if (kind < 0 || kind >= kNumProbes || !buf || !sink || buf_bytes < kProbes[kind].footprint ||
        (reinterpret_cast<uintptr_t>(buf) & 255u) != 0)
        return -1;
    const uint8_t *b = static_cast<const uint8_t *>(buf);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int w = kProbes[kind].wgs;
    switch (kind) {
        case 0: linear_kernel<(size_t)2 << 20, 8><<<w, 256, 0, st>>>(b, sink); break;
        case 1: rows_kernel<5632, 128, 32768, 256><<<w, 256, 0, st>>>(b, sink); break;
        case 2: rows_kernel<5632, 128, 32768, 0><<<w, 256, 0, st>>>(b, sink); break;
        case 3: rows_gemm_order_kernel<5632, 128, 32768, 256><<<w, 256, 0, st>>>(b, sink); break;
        case 4: rows_kernel<1408, 128, 16384, 128><<<w, 256, 0, st>>>(b, sink); break;
        case 5: rows_kernel<1408, 128, 16384, 0><<<w, 256, 0, st>>>(b, sink); break;
        case 6: rows_gemm_order_kernel<1408, 128, 16384, 128><<<w, 256, 0, st>>>(b, sink); break;
        case 7: fused_kernel<<<w, 256, 0, st>>>(b, sink); break;
        default: lds_kernel<<<w, 1024, 0, st>>>(sink); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
