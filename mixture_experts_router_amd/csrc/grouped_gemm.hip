// Grouped expert GEMMs on the gfx950 matrix cores.
//
//   gate/up:  h = gelu_tanh(X W_gate^T) * (X W_up^T)   (GEGLU, Gemma-4-26B-A4B
//             optimisation report, section 1; gelu_pytorch_tanh from the
//             verification report, section 2.1)
//   down:     y = h W_down^T
//
// X for expert e is rows [offsets[e], offsets[e+1]) of the expert-grouped
// order; for gate/up those rows may be gathered straight from x through
// sorted_ids, so the dispatched copy of x is never written to HBM.  The
// grouped matmul of the pages (SwiftGMM, Pangu Pro MoE summary article,
// group 4) is prior art; this is a bf16 MFMA kernel with LDS-staged tiles.
//
// Workgroup = 4 waves = WAVES_M x WAVES_N; tile BM rows x BN columns, K steps
// of 64 staged through double-buffered LDS from registers.  For gate/up the
// BN columns are BN/2 gate rows and the BN/2 matching up rows of the weight,
// laid out so each wave holds gate column n and up column I + n in the same
// lanes and registers, and the GEGLU runs on the fp32 accumulators.
//
// The launch grid is static: blockIdx.x = N tile, blockIdx.y = M-tile slot.
// Each workgroup finds its (expert, row block) from the offsets; slots past
// the last tile exit at once, and an empty expert owns no tile, so its
// weights are never read.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// bf16 bits of an E2M1 code scaled by 2^(sexp): the magnitude (3 bits) is
// 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.  The result is exact when
// it is a normal bf16 number.
__device__ __forceinline__ uint32_t e2m1_to_bf16(uint32_t c, int sexp) {
    const uint32_t m = c & 7u;
    uint32_t bits = (m == 1u) ? (126u << 7) : (((126u + (m >> 1)) << 7) | ((m & 1u) << 6));
    bits = (m == 0u) ? 0u : (uint32_t)((int)bits + (sexp << 7));
    return bits | ((c & 8u) << 12);
}

// Eight codes (low nibble first) and one E8M0 scale byte -> 8 bf16 values.
__device__ __forceinline__ u32x4 dequant8(uint32_t codes, uint32_t sbyte) {
    const int sexp = (int)sbyte - 127;
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = e2m1_to_bf16((codes >> (8 * i)) & 15u, sexp);
        const uint32_t hi = e2m1_to_bf16((codes >> (8 * i + 4)) & 15u, sexp);
        r[i] = lo | (hi << 16);
    }
    return r;
}

struct GemmArgs {
    const uint16_t *a;        // activations: x (gather), x_perm or h
    const int32_t *gather;    // sorted_ids, or nullptr for already-grouped rows
    int gather_k;             // k: row p reads a[gather[p] / k]
    const int32_t *offsets;   // [E + 1]
    const void *w;            // bf16 [E][rows][K] or MXFP4 codes [E][rows][K/2]
    const uint8_t *scales;    // MXFP4 scales [E][rows][K/32] or nullptr
    uint16_t *out;            // [A][n_out] bf16
    int E, K, n_out, I;       // I: gate/up split (gate/up only)
    int w_rows;               // weight rows per expert (2I or H)
};

// Locate this workgroup's M tile: tile index -> (expert, first row).  Run by
// one wave; results go to LDS.
template <int BM>
__device__ __forceinline__ void find_tile(const int32_t *__restrict__ offsets, int E, int tile,
                                          int *s_info) {
    const int lane = threadIdx.x & 63;
    int running = 0;
    bool found = false;
    for (int base = 0; base < E && !found; base += 64) {
        const int e = base + lane;
        int n = 0, off = 0;
        if (e < E) {
            off = offsets[e];
            n = offsets[e + 1] - off;
        }
        const int t = (n + BM - 1) / BM;
        int incl = t;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        const int total = __shfl(incl, 63, 64);
        if (tile < running + total) {
            const int excl = incl - t;
            if (running + excl <= tile && tile < running + incl) {
                s_info[0] = e;
                s_info[1] = (tile - running - excl) * BM;   // first row within the expert
                s_info[2] = n;
                s_info[3] = off;
            }
            found = true;
        }
        running += total;
    }
    if (!found && lane == 0) s_info[0] = -1;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GEGLU, bool MX>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs p) {
    static_assert(WAVES_M * WAVES_N == 4, "four waves");
    constexpr int BK = 64;
    constexpr int WTM = BM / WAVES_M;     // rows per wave
    constexpr int WN = BN / WAVES_N;      // columns per wave
    constexpr int MI = WTM / 16, NI = WN / 16;
    static_assert(MI >= 1 && NI >= 1, "tile too small");
    static_assert(!GEGLU || (NI % 2 == 0), "GEGLU pairs gate and up tiles");
    constexpr int A_CHUNKS = BM * 8;      // 16-byte chunks per A tile
    constexpr int B_CHUNKS = BN * 8;
    constexpr int A_PER = (A_CHUNKS + 255) / 256;
    constexpr int B_PER = (B_CHUNKS + 255) / 256;

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];
    __shared__ int s_info[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (wave == 0) find_tile<BM>(p.offsets, p.E, blockIdx.y, s_info);
    __syncthreads();
    const int e = s_info[0];
    if (e < 0) return;
    const int m0 = s_info[1];
    const int rows = min(BM, s_info[2] - m0);   // valid rows of this tile
    const int seg = s_info[3] + m0;             // global row of tile row 0
    const int K = p.K;
    const int nt = blockIdx.x;

    // ---- per-thread global sources for the A and B chunks
    const uint16_t *a_src[A_PER];
    bool a_ok[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int c = tid + 256 * i;
        const int r = c >> 3, ch = c & 7;
        a_ok[i] = (c < A_CHUNKS) && (r < rows);
        size_t row = 0;
        if (a_ok[i]) row = p.gather ? (size_t)(p.gather[seg + r] / p.gather_k) : (size_t)(seg + r);
        a_src[i] = p.a + row * K + ch * 8;
    }
    const char *b_src[B_PER];
    const uint8_t *s_src[B_PER];
    bool b_ok[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int c = tid + 256 * i;
        const int v = c >> 3, ch = c & 7;
        int wrow;
        bool ok = c < B_CHUNKS;
        if (GEGLU) {
            const int half = WN / 2;
            const int wn = v / WN, within = v % WN;
            const int n = nt * (BN / 2) + wn * half + (within % half);
            ok = ok && n < p.I;
            wrow = within < half ? n : p.I + n;
        } else {
            wrow = nt * BN + v;
            ok = ok && wrow < p.n_out;
        }
        b_ok[i] = ok;
        if (!ok) wrow = 0;
        const size_t rid = (size_t)e * p.w_rows + wrow;
        if (MX) {
            b_src[i] = reinterpret_cast<const char *>(p.w) + rid * (K / 2) + ch * 4;
            s_src[i] = p.scales + rid * (K / 32) + (ch >> 2);
        } else {
            b_src[i] = reinterpret_cast<const char *>(p.w) + (rid * K + ch * 8) * 2;
            s_src[i] = nullptr;
        }
    }

    u32x4 ra[A_PER], rb[B_PER];
    auto load = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4 *>(a_src[i] + kt * BK) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            if (MX) {
                if (b_ok[i]) {
                    const uint32_t codes = *reinterpret_cast<const uint32_t *>(b_src[i] + kt * (BK / 2));
                    const uint32_t sb = s_src[i][kt * (BK / 32)];
                    rb[i] = dequant8(codes, sb);
                } else {
                    rb[i] = u32x4{0, 0, 0, 0};
                }
            } else {
                rb[i] = b_ok[i] ? *reinterpret_cast<const u32x4 *>(b_src[i] + kt * BK * 2) : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int c = tid + 256 * i;
            if (c < A_CHUNKS) {
                const int r = c >> 3, ch = c & 7;
                *reinterpret_cast<u32x4 *>(&As[buf][r * BK + swz(r, ch) * 8]) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int c = tid + 256 * i;
            if (c < B_CHUNKS) {
                const int r = c >> 3, ch = c & 7;
                *reinterpret_cast<u32x4 *>(&Bs[buf][r * BK + swz(r, ch) * 8]) = rb[i];
            }
        }
    };

    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load(kt + 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ch = kk * 4 + (lane >> 4);
            u32x4 af[MI], bfr[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int r = wm * WTM + i * 16 + (lane & 15);
                af[i] = *reinterpret_cast<const u32x4 *>(&As[cur][r * BK + swz(r, ch) * 8]);
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int r = wn * WN + j * 16 + (lane & 15);
                bfr[j] = *reinterpret_cast<const u32x4 *>(&Bs[cur][r * BK + swz(r, ch) * 8]);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < KT) store(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    const int col = lane & 15, rq = (lane >> 4) * 4;
    if (GEGLU) {
        constexpr int HALF_T = NI / 2;
#pragma unroll
        for (int j = 0; j < HALF_T; ++j) {
            const int n = nt * (BN / 2) + wn * (WN / 2) + j * 16 + col;
            if (n >= p.I) continue;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = wm * WTM + i * 16 + rq + q;
                    if (r < rows) {
                        const float g = acc[i][j][q], u = acc[i][j + HALF_T][q];
                        p.out[(size_t)(seg + r) * p.n_out + n] = (uint16_t)f32_to_bf16_rne(gelu_tanh(g) * u);
                    }
                }
        }
    } else {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int n = nt * BN + wn * WN + j * 16 + col;
            if (n >= p.n_out) continue;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = wm * WTM + i * 16 + rq + q;
                    if (r < rows) p.out[(size_t)(seg + r) * p.n_out + n] = (uint16_t)f32_to_bf16_rne(acc[i][j][q]);
                }
        }
    }
}

// Upper bound on the number of M tiles: sum_e ceil(n_e / BM) with
// sum_e n_e = A and at most min(E, A) non-empty experts.
static int mtile_slots(int A, int E, int BM) {
    const long long ne = A < E ? A : E;
    return (int)(((long long)A + (long long)(BM - 1) * ne) / BM);
}

template <int BM, int BN, int WM, int WN, bool GEGLU, bool MX>
static hipError_t launch_cfg(const GemmArgs &a, int A, hipStream_t st) {
    const int ncols = GEGLU ? a.I : a.n_out;
    const int per_tile = GEGLU ? BN / 2 : BN;
    dim3 grid((ncols + per_tile - 1) / per_tile, mtile_slots(A, a.E, BM));
    if (grid.y == 0) return hipSuccess;
    grouped_gemm_kernel<BM, BN, WM, WN, GEGLU, MX><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

// Row-block size from the mean rows per expert (a function of the shape
// only, so the launch does not depend on the routing).
template <bool GEGLU, bool MX>
static hipError_t launch_sized(const GemmArgs &a, int A, hipStream_t st) {
    const int mean_rows = A / a.E;
    if (mean_rows <= 16) return launch_cfg<16, 128, 1, 4, GEGLU, MX>(a, A, st);
    if (mean_rows <= 48) return launch_cfg<32, 128, 2, 2, GEGLU, MX>(a, A, st);
    if (mean_rows <= 96) return launch_cfg<64, 128, 2, 2, GEGLU, MX>(a, A, st);
    return launch_cfg<128, 128, 2, 2, GEGLU, MX>(a, A, st);
}

hipError_t launch_gateup(const uint16_t *x, const int32_t *sorted_ids, int k, const int32_t *offsets,
                         const void *w, const uint8_t *scales, uint16_t *h, int A, int H, int E, int I,
                         bool mx, hipStream_t st) {
    GemmArgs a{x, sorted_ids, k, offsets, w, scales, h, E, H, I, I, 2 * I};
    return mx ? launch_sized<true, true>(a, A, st) : launch_sized<true, false>(a, A, st);
}

hipError_t launch_down(const uint16_t *h, const int32_t *offsets, const void *w, const uint8_t *scales,
                       uint16_t *y, int A, int H, int E, int I, bool mx, hipStream_t st) {
    GemmArgs a{h, nullptr, 1, offsets, w, scales, y, E, I, H, I, H};
    return mx ? launch_sized<false, true>(a, A, st) : launch_sized<false, false>(a, A, st);
}

}  // namespace moe
