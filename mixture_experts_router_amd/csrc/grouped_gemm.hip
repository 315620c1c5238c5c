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
// group 4) is prior art only.
//
// Workgroup = 4, 8 or 16 waves = WAVES_M (token direction) x WAVES_N (weight-row
// direction); tile BM tokens x BN weight rows, K in steps of BK.  Operand
// tiles go straight from global memory into LDS (global_load_lds_dwordx4,
// issued from inline asm so that the compiler adds no waits of its own) in
// rings of NS token stages and NS or NS + 1 weight stages; each wave waits
// only for its own loads (explicit vmcnt) and a barrier publishes a stage.
// With the deeper weight ring a wave's weight loads are spread among its
// MFMAs.  The MFMA takes the weight tile as its A
// operand and the tokens as B, so each lane ends with four consecutive output
// columns of one token; the epilogue pairs fragments across lanes (a lane
// swap) so that a lane stores eight consecutive columns.
//
// For gate/up the BN weight rows of a tile are BN/2 gate rows and the BN/2
// matching up rows, interleaved per wave so that gate column n and up column
// I + n land in the same lane and register; the GEGLU runs on the fp32
// accumulators.  4-bit weights (MXFP4, NVFP4) stay packed in LDS and are
// expanded to exact bf16 when each fragment is read; W4A4 multiplies packed
// MXFP4 operands on the block-scaled FP4 MFMA.  The router for many tokens
// runs on the same engine (one dense group, fp32 chunk sums added in fp64).
//
// The launch grid is static (one dimension, N tiles x M-tile slots, dealt
// to the XCDs in groups).  Each workgroup finds its (expert, row block) from
// the offsets; slots past the last tile exit at once, an empty expert owns no
// tile (its weights are never read), and waves whose rows all lie past the
// expert's last row skip their MFMAs.
#include <type_traits>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct GemmArgs {
    const uint16_t *a;        // activations: x (gather), x_perm or h
    const int32_t *gather;    // sorted_ids, or nullptr for already-grouped rows
    int gather_k;             // k: row p reads a[gather[p] / k]
    const int32_t *offsets;   // [E + 1]
    const void *w;            // bf16 [E][rows][K] or MXFP4 codes [E][rows][K/2]
    const uint8_t *scales;    // MXFP4 scales [E][rows][K/32], NVFP4 [E][rows][K/16], or nullptr
    uint16_t *out;            // [A][n_out] bf16
    int E, K, n_out, I;       // I: gate/up split (gate/up only)
    int w_rows;               // weight rows per expert (2I or H)
    int n_tiles;              // N tiles per M tile
    int stream_max_rows;      // experts with at most this many rows stream their weights
    // dense router mode: one group of `dense_rows` tokens, fp32 output
    int dense_rows;
    float *out32;             // [T][E] logits
    const float *bias;        // [E] or nullptr
    // Optional always-on group (a dense GEGLU MLP run as a shared expert):
    // its tiles follow the first `routed_blocks` blocks; its rows are all
    // sh_rows tokens in order (no gather), with its own operands and sizes.
    int routed_blocks;
    int sh_rows;              // 0: no shared group
    int sh_n_tiles;           // N tiles per M tile of the shared group
    const uint16_t *sh_a;     // [sh_rows][sh_K]
    const void *sh_w;         // [sh_w_rows][sh_K] bf16, or MXFP4 codes
    const uint8_t *sh_scales; // [sh_w_rows][sh_K / 32] or nullptr
    uint16_t *sh_out;         // [sh_rows][sh_n_out] bf16 (gate/up)
    float *sh_out32;          // [sh_splits][sh_rows][sh_n_out] fp32 partial sums (down)
    int sh_K, sh_I, sh_w_rows, sh_n_out;
    int sh_splits, sh_ksplit; // down: K cut into sh_splits ranges of sh_ksplit (last one shorter)
    // W4A4: `a` holds MXFP4 codes [rows][K/2] and a_scales [rows][K/32]
    const uint8_t *a_scales;
    // NVFP4 weights: `scales` holds E4M3 codes [E][rows][K/16] and w_global
    // the fp32 scale of each expert's matrix [E]; with NVFP4 activations,
    // a_global points at their fp32 input scale (the activations arrive
    // decoded without it), else nullptr
    const float *w_global;
    const float *a_global;
    // Row-tile groups run last to first on each XCD (large row blocks only)
    int reverse_groups;
    // Routed output rows: grouped row r is stored at out row out_rows[r]
    // (the down GEMM of the whole layer passes sorted_ids, so y lands in
    // (token, slot) order), or at row r when nullptr
    const int32_t *out_rows;
    // Buffer extents in bytes, for the bounds checks of the MOE_DEBUG build:
    // the routed group's (or the router's) operands and output, then the
    // shared group's.
    size_t a_bytes, gather_bytes, w_bytes, s_bytes, out_bytes, a_s_bytes, out_rows_bytes;
    size_t sh_a_bytes, sh_w_bytes, sh_s_bytes, sh_out_bytes;
};

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts by 1,
// 2, 4 and 8 sum within each row of 16 lanes, then the last lane of row 0
// is added to row 1 and of row 2 to row 3 (row_bcast:15), and the last lane
// of row 1 (by then rows 0 and 1) to rows 2 and 3 (row_bcast:31).  Lanes
// whose source lies outside the row, or whose row is masked off, add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Locate this workgroup's M tile: tile index -> (expert e, first row m0
// within the expert, the expert's rows n and its first grouped row off), or
// e = -1 past the last tile: a wave prefix scan of ceil(n_e / BM) over the
// experts, 64 at a time (their offsets requested 256 at a time, so the
// layer's 128 experts cost one memory round trip); the results are
// wave-uniform.  Measured against a shuffle scan that loaded 64 offsets per
// round trip: the 256-row down tiles of 2048-8192 tokens 2-3% faster, the
// decode step 0.7 us.
struct TileInfo {
    int e, m0, n, off;
};
template <int BM>
__device__ __forceinline__ TileInfo find_tile(const int32_t *__restrict__ offsets, int E, int tile) {
    const int lane = threadIdx.x & 63;
    constexpr int PRE = 4;   // chunks of 64 experts whose offsets are requested together
    int running = 0;
    for (int base0 = 0; base0 < E; base0 += 64 * PRE) {
        int lo[PRE], hi[PRE];
#pragma unroll
        for (int c = 0; c < PRE; ++c) {
            const int e = base0 + 64 * c + lane;
            lo[c] = e < E ? offsets[e] : 0;
            hi[c] = e < E ? offsets[e + 1] : 0;
        }
#pragma unroll
        for (int c = 0; c < PRE; ++c) {
            const int base = base0 + 64 * c;
            if (base >= E) break;
            const int n = hi[c] - lo[c], off = lo[c];
            const int t = (n + BM - 1) / BM;
            const int incl = wave_incl_scan(t);
            const int total = __builtin_amdgcn_readlane(incl, 63);
            if (tile < running + total) {
                const int excl = incl - t;
                const uint64_t hit = __ballot(running + excl <= tile && tile < running + incl);
                const int src = (int)__builtin_ctzll(hit);   // the expert holding the tile
                TileInfo r;
                r.e = base + src;
                r.n = __builtin_amdgcn_readlane(n, src);
                r.off = __builtin_amdgcn_readlane(off, src);
                r.m0 = (tile - running - __builtin_amdgcn_readlane(excl, src)) * BM;
                return r;
            }
            running += total;
        }
    }
    return TileInfo{-1, 0, 0, 0};
}

enum GemmMode { kDown = 0, kGateUp = 1, kRouter = 2 };

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE, bool MX, int NS_, int BK_, bool A4_ = false,
          bool NV_ = false, bool WD_ = false, int NSB_ = 0>
struct GemmTile {
    static constexpr bool GEGLU = MODE == kGateUp;
    static constexpr int BK = BK_;                // K per step (32, 64, 128; 4-bit weights 64 or 256)
    static constexpr int CH = BK / 8;             // 16-byte chunks per tile row
    static constexpr int RPD = 64 / CH;           // tile rows per 1 KB direct-to-LDS load
    static constexpr int KK = BK / 32;            // MFMA K steps per step
    static constexpr int NS = NS_;                // LDS stages (NS - 1 loads ahead) of the token tile
    // Stages of the weight tile: NS, or one more in the bf16 256 x 256 tile
    // (two token stages and three weight stages fill the 160 KB of LDS): the
    // weights come from HBM, the token rows mostly from L2, so the weights
    // are requested one step earlier.
    static constexpr int NSB = NSB_ ? NSB_ : NS_;
    static constexpr int NW = WAVES_M * WAVES_N;   // waves per workgroup
    static constexpr int NT = 64 * NW;             // threads per workgroup
    static constexpr int WTM = BM / WAVES_M;      // tokens per wave
    static constexpr int WN = BN / WAVES_N;       // weight rows per wave
    static constexpr int MI = WTM / 16;           // token tiles per wave (MFMA B operand)
    static constexpr int NI = WN / 16;            // weight-row tiles per wave (MFMA A operand)
    // Direct-to-LDS loads move 1 KB per wave instruction (64 lanes x 16 B):
    // RPD rows of BK bf16.
    static constexpr int SC_BLK = NV_ ? 16 : 32;                 // 4-bit weights: K values per block scale
    static constexpr int SC_PER = BK / SC_BLK;                   // scale bytes per row and step
    // 4-bit weights in 256-wide steps go straight to LDS like the tokens:
    // code rows of 128 bytes (8 rows per 1 KB load) and their scale bytes
    // (4 bytes per lane, [row][SC_PER] in LDS).  With WD_ (64-wide steps)
    // the code rows of 32 bytes go straight to LDS too (32 rows per load)
    // and the tile's block scales, whole rows of K/32 (MXFP4) or K/16
    // (NVFP4) bytes, are read into LDS once when the tile starts.
    // Otherwise, in 64-wide steps, they are staged through registers.
    static constexpr bool WDMA = MX && (BK == 256 || WD_);
    static constexpr bool SC_TILE = WDMA && BK == 64;      // scales of the whole K range, per tile
    static constexpr int SC_ROW = NV_ ? 176 : 100;         // LDS bytes per scale row (K <= 2816 / 3200)
    static constexpr int CRB = BK / 2;                     // bytes per code row and step
    static constexpr int CCH = CRB / 16;                   // 16-byte chunks per code row
    static constexpr int CROWS = 1024 / CRB;               // code rows per 1 KB load
    static constexpr int NA = BM / RPD;           // token-tile instructions per stage
    static constexpr int NB = MX ? (WDMA ? BN / CROWS : 0) : BN / RPD;   // weight-tile instructions per stage
    static constexpr int NSC = WDMA && !SC_TILE ? BN * SC_PER / 256 : 0;   // scale instructions per stage
    static constexpr int A_W = (NA + NW - 1) / NW;   // per wave (upper bound)
    static constexpr int B_W = (NB + NW - 1) / NW;
    static constexpr int S_W = (NSC + NW - 1) / NW;
    // MXFP4 / NVFP4 weights through registers: BN rows x BK/32 chunks of 16
    // bytes (BK codes) plus their block scales (BK/32 E8M0 or BK/16 E4M3
    // bytes).
    static constexpr int CPR = BK / 32;           // 16-byte code chunks per row and step
    static constexpr int MB_CHUNKS = MX && !WDMA ? BN * CPR : 0;
    static constexpr int MB_PER = MB_CHUNKS ? (MB_CHUNKS + NT - 1) / NT : 1;
    static constexpr int MS_PER = MX && !WDMA ? (BN + NT - 1) / NT : 1;
    static constexpr int A_LDS = BM * BK;                      // uint16 per stage
    static constexpr int B_LDS = MX ? BN * BK / 4 : BN * BK;   // uint16 per stage
    static_assert(NW == 4 || NW == 8 || NW == 16, "four, eight or sixteen waves");
    static_assert(MI >= 1 && NI >= 1, "tile too small");
    static_assert(!GEGLU || (NI % 2 == 0), "GEGLU pairs gate and up tiles");
    static_assert(BK == 32 || BK == 64 || BK == 128 || ((MX || MODE == kRouter) && BK == 256), "K step");
    static_assert(BM % RPD == 0 && BN % RPD == 0, "whole 1 KB load groups");
    static_assert(!MX || BK == 64 || BK == 256, "4-bit weight tiles use K steps of 64 or 256");
    static_assert(NS >= 2 && NS <= 8, "stages");
    // MXFP4 codes go through registers one step ahead; the wait counts
    // assume at most one DMA step is issued after them.
    static_assert(!MX || WDMA || NS <= 3, "MXFP4 pipeline depth");
    static_assert(!WDMA || (BN % CROWS == 0 && (SC_TILE || (BN * SC_PER) % 256 == 0)), "whole 4-bit load groups");
    static_assert(!WD_ || (MX && BK == 64), "per-tile scales: 4-bit weights in 64-wide steps");
    // W4A4: both operands are MXFP4 codes loaded like bf16 tiles (128-byte
    // rows = 256 K values per stage, two 16x16x128 scaled MFMA steps).
    static_assert(!A4_ || (!MX && BK == 64), "W4A4 tiles: code rows of 128 bytes");
    // NVFP4 weights take the MXFP4 route with an E4M3 scale per 16 K values
    // (kept in LDS as bytes, decoded where a fragment uses it)
    static_assert(!NV_ || (MX && !A4_), "NVFP4 is a variant of the MXFP4 weight path");
    static constexpr int SCW = SC_PER >= 4 ? SC_PER / 4 : 1;     // scale bytes per row and step in 32-bit words
    static constexpr int SS_BYTES = SC_TILE ? SC_ROW * BN : MX ? SC_PER * BN : 0;
    static constexpr int SS_SLOTS = SC_TILE ? 1 : NSB;   // per-tile scales: one buffer
    // W4A4 block scales of a stage: 8 bytes (blocks 8 kt .. 8 kt + 7) per
    // weight row and per token row, one row per thread.
    static constexpr bool SC_PAIR_M = MI >= 2;   // token rows paired like weight rows
    static constexpr int SC_W = ((BN + 31) / 32) * 32 * 8;
    static constexpr int SC_BYTES = SC_W + (SC_PAIR_M ? ((BM + 31) / 32) * 32 : BM) * 8;
    static_assert(!A4_ || BN + BM <= NT, "W4A4: one scale row per thread");
    // the scale stores wait for all of the wave's loads (the compiler cannot
    // count the direct-to-LDS ones), which only a two-stage pipeline affords
    static_assert(!A4_ || NS == 2, "W4A4: two stages");
    static_assert(!A4_ || (NI % 2 == 0 && (!SC_PAIR_M || MI % 2 == 0)), "W4A4: scale rows in pairs");
    // a deeper weight ring: two token stages and three or more weight stages
    // (bf16 tiles, or 4-bit codes straight to LDS)
    static_assert(NSB == NS || (NS == 2 && NSB >= 3 && !A4_ && (!MX || WDMA)), "weight ring deeper than the token ring");
    // LDS: token stages, weight stages, block scales (4-bit weights), W4A4
    // scale pairs, carved from one buffer (byte offsets, 16-byte aligned)
    static constexpr int A_OFF = 0;
    static constexpr int B_OFF = A_OFF + NS * A_LDS * 2;
    static constexpr int S_OFF = B_OFF + NSB * B_LDS * 2;
    static constexpr int C_OFF = S_OFF + ((SS_SLOTS * SS_BYTES + 15) / 16) * 16;
    static constexpr int I_OFF = C_OFF + ((A4_ ? NS * SC_BYTES : 0) + 15) / 16 * 16;
    // The tile lookup runs in wave 0 and reaches the others through 16 bytes
    // of LDS where they fit; a tile that fills the 160 KB runs it in every
    // wave instead.
    static constexpr bool INFO_LDS = I_OFF + 16 <= 160 * 1024;
    static constexpr int LDS_BYTES = I_OFF + (INFO_LDS ? 16 : 0);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");
};

// s_waitcnt with vmcnt = VM and lgkmcnt = 0 (expcnt left at its maximum).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// The same for a wave-uniform count known only at run time (0..31; larger
// counts wait for everything, which is always safe).
__device__ __forceinline__ void wait_vm_lgkm0_rt(int n) {
    switch (n) {
#define MOE_WAIT_CASE(N) \
    case N: wait_vm_lgkm0<N>(); break;
        MOE_WAIT_CASE(1) MOE_WAIT_CASE(2) MOE_WAIT_CASE(3) MOE_WAIT_CASE(4) MOE_WAIT_CASE(5)
        MOE_WAIT_CASE(6) MOE_WAIT_CASE(7) MOE_WAIT_CASE(8) MOE_WAIT_CASE(9) MOE_WAIT_CASE(10)
        MOE_WAIT_CASE(11) MOE_WAIT_CASE(12) MOE_WAIT_CASE(13) MOE_WAIT_CASE(14) MOE_WAIT_CASE(15)
        MOE_WAIT_CASE(16) MOE_WAIT_CASE(17) MOE_WAIT_CASE(18) MOE_WAIT_CASE(19) MOE_WAIT_CASE(20)
        MOE_WAIT_CASE(21) MOE_WAIT_CASE(22) MOE_WAIT_CASE(23) MOE_WAIT_CASE(24) MOE_WAIT_CASE(25)
        MOE_WAIT_CASE(26) MOE_WAIT_CASE(27) MOE_WAIT_CASE(28) MOE_WAIT_CASE(29) MOE_WAIT_CASE(30)
        MOE_WAIT_CASE(31)
#undef MOE_WAIT_CASE
        default: wait_vm_lgkm0<0>(); break;
    }
}

// 16-byte direct global->LDS load of one wave: lane l's 16 bytes from `g`
// land at lds + 16 l.  Issued from inline asm so that the compiler adds no
// waits of its own on later LDS reads (it cannot tell the stage buffers
// apart); every wait is the explicit s_waitcnt of the pipeline below.  The
// asm has no register outputs, and M0 is only ever set here.
// STREAM sets the non-temporal hint, for data read exactly once: on gfx950 a
// streaming read of whole lines with the hint reaches about 10% more HBM
// bandwidth (measured: 6.8 vs 6.1 TB/s for a 2 GiB read).  Data that other
// workgroups re-read, or lines consumed in pieces over several K steps (the
// 32-byte MXFP4 row slices), lose more from the early eviction than they gain.
// The compiler reserves M0 and ignores it in a clobber list (it warns so);
// nothing it generates in these kernels keeps a value in M0 (no LDS-DMA,
// GWS, message or relative-move builtins are used), so setting it inside
// the asm is safe, and the warning is silenced for these two helpers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool STREAM>
__device__ __forceinline__ void dma16(const void *g, const void *lds) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    if (STREAM)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(l) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(l) : "memory", "m0");
}

// Epilogue exchange between lanes l and l ^ 16 (k groups lk and lk ^ 1, which
// hold columns 4 lk .. 4 lk + 3 of the same output row): a lane of an even
// group keeps fragment 0's four values and receives its partner's, a lane of
// an odd group receives the partner's fragment-1 values and keeps its own,
// so each lane ends with 8 consecutive columns of one fragment.
__device__ __forceinline__ uint4 pair_swap16(uint2 f0, uint2 f1, int odd) {
    const uint2 keep = odd ? f1 : f0, send = odd ? f0 : f1;
    // v_permlane16_swap exchanges the odd 16-lane rows of its first operand
    // with the even rows of its second: with both operands the same value,
    // an even row finds its partner's value in the second result, an odd
    // row in the first
    const auto rx = __builtin_amdgcn_permlane16_swap(send.x, send.x, false, false);
    const auto ry = __builtin_amdgcn_permlane16_swap(send.y, send.y, false, false);
    const uint2 recv = odd ? make_uint2(rx[0], ry[0]) : make_uint2(rx[1], ry[1]);
    return odd ? make_uint4(recv.x, recv.y, keep.x, keep.y) : make_uint4(keep.x, keep.y, recv.x, recv.y);
}

// 4-byte direct global->LDS load of one wave: lane l's 4 bytes from `g`
// land at lds + 4 l (same rules as dma16).
__device__ __forceinline__ void dma4(const void *g, const void *lds) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(l) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE, bool MX, int NS_, int BK_, bool A4 = false,
          bool NV = false, bool WD = false, int NSB_ = 0>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void grouped_gemm_kernel(GemmArgs p) {
    using G = GemmTile<BM, BN, WAVES_M, WAVES_N, MODE, MX, NS_, BK_, A4, NV, WD, NSB_>;
    constexpr bool GEGLU = MODE == kGateUp, ROUTER = MODE == kRouter;
    constexpr int BK = G::BK, NS = G::NS, NSB = G::NSB, WTM = G::WTM, WN = G::WN, MI = G::MI, NI = G::NI;
    constexpr int CH = G::CH, RPD = G::RPD, KK = G::KK;
    constexpr int NA = G::NA, NB = G::NB, A_W = G::A_W, B_W = G::B_W, NW = G::NW, NT = G::NT;

    // bf16 tiles: [row][BK/8 chunks of 16 B], chunk index XOR-swizzled by row.
    // 4-bit weights through registers: codes [word of 8 codes][row], scale
    // bytes [block][row]; straight to LDS in 256-wide steps: codes [row][8
    // chunks of 16 B] (XOR-swizzled by row & 7), scale bytes [row][block];
    // in 64-wide steps: codes [row][2 chunks] (XOR-swizzled by (row >> 3) &
    // 1), scale bytes of the whole K range [row][SC_ROW].
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::LDS_BYTES];
    uint16_t(*As)[G::A_LDS] = reinterpret_cast<uint16_t(*)[G::A_LDS]>(smem + G::A_OFF);   // [NS]
    uint16_t(*Bs)[G::B_LDS] = reinterpret_cast<uint16_t(*)[G::B_LDS]>(smem + G::B_OFF);   // [NSB]
    constexpr int SSB = G::SS_BYTES > 0 ? G::SS_BYTES : 1, SCB = A4 ? G::SC_BYTES : 1;
    uint8_t(*Ss)[SSB] = reinterpret_cast<uint8_t(*)[SSB]>(smem + G::S_OFF);               // [SS_SLOTS]
    uint8_t(*Sc)[SCB] = reinterpret_cast<uint8_t(*)[SCB]>(smem + G::C_OFF);               // [NS], W4A4

    // XCD-aware tile order.  Workgroups go to the 8 XCDs round-robin (block
    // b -> XCD b % 8).  The N tiles of one M tile form a group that shares
    // its token rows; groups are dealt to XCDs round-robin (group m -> XCD
    // m % 8) and each XCD runs its groups in order, so a group's token rows
    // stay in one XCD's L2 while the empty slots at the end of the grid are
    // spread evenly over the XCDs.
    // With reverse_groups each XCD runs its groups last to first (group m
    // still on XCD m % 8).
    // Small row blocks share little: there the plain order (N tile fastest)
    // spreads each expert's weight slabs over all XCDs.
    // Shared-group tiles come after the routed ones, in plain order.
    const bool shared = !ROUTER && p.sh_rows > 0 && (int)blockIdx.x >= p.routed_blocks;
    int mslot, nt;
    int split = 0;
    if (shared) {
        const int idx = blockIdx.x - p.routed_blocks;
        const int per_split = ((p.sh_rows + BM - 1) / BM) * p.sh_n_tiles;
        split = idx / per_split;
        mslot = (idx % per_split) / p.sh_n_tiles;
        nt = idx % p.sh_n_tiles;
    } else if (BM >= 64) {
        const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
        const int grp = j / p.n_tiles, ngrp = p.routed_blocks / p.n_tiles / 8;   // groups per XCD
        mslot = xcd + 8 * (p.reverse_groups ? ngrp - 1 - grp : grp);
        nt = j % p.n_tiles;
    } else {
        mslot = blockIdx.x / p.n_tiles;
        nt = blockIdx.x % p.n_tiles;
    }
    // This tile's group: operands and sizes (block-uniform).
    const uint16_t *g_a = shared ? p.sh_a : p.a;
    const int32_t *g_gather = shared ? nullptr : p.gather;
    const void *g_w = shared ? p.sh_w : p.w;
    const uint8_t *g_scales = shared ? p.sh_scales : p.scales;
    uint16_t *g_out = shared ? p.sh_out : p.out;
    const int g_I = shared ? p.sh_I : p.I;
    const int g_w_rows = shared ? p.sh_w_rows : p.w_rows;
    const int g_n_out = shared ? p.sh_n_out : p.n_out;
    [[maybe_unused]] const size_t g_a_bytes = shared ? p.sh_a_bytes : p.a_bytes;
    [[maybe_unused]] const size_t g_w_bytes = shared ? p.sh_w_bytes : p.w_bytes;
    [[maybe_unused]] const size_t g_s_bytes = shared ? p.sh_s_bytes : p.s_bytes;
    [[maybe_unused]] const size_t g_out_bytes = shared ? p.sh_out_bytes : p.out_bytes;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    int e, m0, rows, seg;
    bool stream = false;   // this tile is the only reader of its weight slab
    if (ROUTER) {                               // one dense group of tokens
        if (mslot * BM >= p.dense_rows) return;
        e = 0;
        m0 = mslot * BM;
        rows = min(BM, p.dense_rows - m0);
        seg = m0;
    } else if (shared) {                        // every token, in order
        e = 0;
        m0 = mslot * BM;
        rows = min(BM, p.sh_rows - m0);
        seg = m0;
        stream = p.sh_rows <= p.stream_max_rows;
    } else {
        TileInfo ti;
        if constexpr (G::INFO_LDS) {
            int *s_info = reinterpret_cast<int *>(smem + G::I_OFF);
            if (wave == 0) {
                ti = find_tile<BM>(p.offsets, p.E, mslot);
                if (lane == 0) {
                    s_info[0] = ti.e;
                    s_info[1] = ti.m0;
                    s_info[2] = ti.n;
                    s_info[3] = ti.off;
                }
            }
            __syncthreads();
            ti = TileInfo{s_info[0], s_info[1], s_info[2], s_info[3]};
        } else {
            ti = find_tile<BM>(p.offsets, p.E, mslot);
        }
        e = __builtin_amdgcn_readfirstlane(ti.e);
        if (e < 0) return;
        m0 = __builtin_amdgcn_readfirstlane(ti.m0);
        const int n_e = __builtin_amdgcn_readfirstlane(ti.n);
        rows = min(BM, n_e - m0);                                         // valid tokens of this tile
        seg = __builtin_amdgcn_readfirstlane(ti.off) + m0;                // global row of tile token 0
        stream = n_e <= p.stream_max_rows;
    }
    const int K = shared ? p.sh_K : p.K;                 // row length of both operands
    const int kb = shared ? split * p.sh_ksplit : 0;     // this tile's K range [kb, kb + KT*BK)
    // W4A4 rows hold K/2 bytes of codes (K/4 16-bit units) and a stage holds
    // 256 K values; a last stage that runs past the row is masked (below).
    const int rowu = A4 ? K / 4 : K;                     // row length in 16-bit units
    // 4-bit weights straight to LDS (256-wide steps) also end with a partial
    // stage when K is not a multiple of 256.
    const int KT = A4 || (G::WDMA && BK == 256) ? (K + 255) / 256
                                                : (shared && p.sh_splits > 1 ? min(p.sh_ksplit, K - kb) : K) / BK;

    // Weight row of tile row v (0 <= v < BN), clamped to a valid row.
    auto weight_row = [&](int v) -> int {
        if (GEGLU) {
            const int half = WN / 2;
            const int wn = v / WN, within = v % WN;
            const int n = nt * (BN / 2) + wn * half + (within % half);
            return n < g_I ? (within < half ? n : g_I + n) : 0;
        }
        const int r = nt * BN + v;
        return r < g_n_out ? r : 0;
    };

    // ---- direct-to-LDS sources.  Instruction g fills rows RPD*g .. RPD*g +
    // RPD - 1 of the stage buffer; lane l lands at row RPD*g + l/CH, physical
    // chunk l%CH, so it fetches logical chunk (l%CH) ^ swizzle(row).  A token
    // row past the tile's end reads the tile's first row and a weight row
    // past the matrix reads row 0; both only feed outputs never stored.
    const int lr = lane / CH, lc = lane % CH;
    const uint16_t *a_src[A_W];
    int a_ch[G::WDMA ? A_W : 1];   // 4-bit weight path: the lane's chunk column, clamped per step
#pragma unroll
    for (int q = 0; q < A_W; ++q) {
        const int g = q * NW + wave;
        const int row = RPD * (g < NA ? g : 0) + lr;
        const int rr = row < rows ? row : 0;
        const size_t src = g_gather ? (size_t)(*MOE_CHECKED(g_gather + seg + rr, 4, g_gather, p.gather_bytes) /
                                               p.gather_k)
                                    : (size_t)(seg + rr);
        if (G::WDMA) {
            a_src[q] = g_a + src * rowu + kb;
            a_ch[q] = 8 * tswz<BK>(row, lc);
        } else {
            a_src[q] = g_a + src * rowu + kb + (A4 ? 0 : 8 * tswz<BK>(row, lc));
        }
    }
    constexpr bool WDMA = G::WDMA;
    const uint16_t *b_src[B_W > 0 ? B_W : 1];
#pragma unroll
    for (int q = 0; q < B_W; ++q) {
        const int g = q * NW + wave;
        if (WDMA) {   // CROWS code rows of CRB bytes: lane l -> row CROWS g + l / CCH, chunk l % CCH (swizzled)
            const int row = G::CROWS * (g < NB ? g : 0) + lane / G::CCH;
            const size_t rid = (size_t)e * g_w_rows + weight_row(row);
            b_src[q] = reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(g_w) + rid * (K / 2) + kb / 2);
        } else {
            const int row = RPD * (g < NB ? g : 0) + lr;
            const size_t rid = (size_t)e * g_w_rows + weight_row(row);
            b_src[q] = reinterpret_cast<const uint16_t *>(g_w) + rid * rowu + kb + (A4 ? 0 : 8 * tswz<BK>(row, lc));
        }
    }
    // Weight load groups that hold a valid output column.  A group lies in
    // one half (gate or up) of one wave's rows, so its first row decides;
    // groups wholly past the last column (the half-filled last column tile
    // of the gate/up when I is not a multiple of BN / 2) are not loaded
    // (measured at 2048 tokens, MXFP4 gate/up with I = 704: 202 -> 195 us).
    bool b_on[B_W > 0 ? B_W : 1];
#pragma unroll
    for (int q = 0; q < B_W; ++q) {
        const int g = q * NW + wave;
        const int v0 = (WDMA ? G::CROWS : RPD) * g;
        const bool valid_col = GEGLU ? nt * (BN / 2) + (v0 / WN) * (WN / 2) + (v0 % WN) % (WN / 2) < g_I
                                     : nt * BN + v0 < g_n_out;
        b_on[q] = (NB % NW == 0 || g < NB) && valid_col;
    }
    // Scale rows of direct-loaded 4-bit weights: SC_PER bytes per row and
    // step, 4 per lane, 256 / SC_PER rows per load.
    const uint8_t *s_src[G::S_W > 0 ? G::S_W : 1];
#pragma unroll
    for (int q = 0; q < G::S_W; ++q) {
        constexpr int LPR = G::SC_PER >= 4 ? G::SC_PER / 4 : 1;   // lanes per row (used with SC_PER >= 4)
        const int g = q * NW + wave;
        const int row = (256 / G::SC_PER) * (g < G::NSC ? g : 0) + lane / LPR;
        const size_t rid = (size_t)e * g_w_rows + weight_row(row);
        s_src[q] = g_scales + rid * (K / G::SC_BLK) + kb / G::SC_BLK;
    }
    // The lane's logical code chunk (the same in every load group: 128-byte
    // rows, 8 to a group, XOR row & 7, which is lane / 8; 32-byte rows, 32
    // to a group, XOR (row >> 3) & 1, which is (lane >> 4) & 1) and scale
    // word.  Past the row's end (the last, partial stage of 256-wide steps)
    // the loads re-read the row's last chunk / scale word; those code chunks
    // are then zeroed in LDS (zero_tail_w), so they multiply as zeros.
    const int w_ch = G::CCH == 8 ? (lane & 7) ^ ((lane >> 3) & 7) : (lane & 1) ^ ((lane >> 4) & 1);
    const int s_word = G::WDMA ? 4 * (lane % (G::SC_PER >= 4 ? G::SC_PER / 4 : 1)) : 0;
    auto wcol_bytes = [&](int kt) { return min(kt * G::CRB + 16 * w_ch, K / 2 - 16); };
    auto scol_bytes = [&](int kt) { return min(kt * G::SC_PER + s_word, K / G::SC_BLK - 4); };
    // W4A4: the lane's 16-byte chunk within a stage (the same for every load
    // group: a group covers 8 rows, so row & 7 == lr), clamped into the row
    // for the last, partial stage.
    const int lane_col = 8 * tswz<BK>(lr, lc);
    auto col_of = [&](int kt) -> int {
        if (!A4) return kt * BK;
        return min(kt * BK + lane_col, rowu - 8);
    };
    // Token-row groups past the tile's last valid row are not loaded (their
    // LDS rows keep stale data that only reaches outputs never stored).
    const int na_valid = (rows + RPD - 1) / RPD;
    // Token tile of step kt into stage kt % NS.
    auto issue_a = [&](int kt) {
        const int slot = kt % NS;
#pragma unroll
        for (int q = 0; q < A_W; ++q) {
            const int g = q * NW + wave;
            if (g < na_valid) {
                if (G::WDMA)
                    dma16<false>(MOE_CHECKED(a_src[q] + min(kt * BK + a_ch[q], K - 8), 16, g_a, g_a_bytes),
                                 As[slot] + g * 512);
                else
                    dma16<false>(MOE_CHECKED(a_src[q] + col_of(kt), 16, g_a, g_a_bytes), As[slot] + g * 512);
            }
        }
    };
    // Weight load q of this wave for step kt, into stage kt % NSB.
    auto issue_bq = [&](int kt, int q) {
        const int slot = kt % NSB;
        const int bcol = WDMA ? wcol_bytes(kt) / 2 : col_of(kt);   // in 16-bit units
        const int g = q * NW + wave;
        if (b_on[q]) {
            // Weights of an expert with one row tile are read once: stream
            // them past the caches.  Several row tiles re-read them: keep.
            if (stream)
                dma16<true>(MOE_CHECKED(b_src[q] + bcol, 16, g_w, g_w_bytes), Bs[slot] + g * 512);
            else
                dma16<false>(MOE_CHECKED(b_src[q] + bcol, 16, g_w, g_w_bytes), Bs[slot] + g * 512);
        }
    };
    // Weight tile (and block scales) of step kt.
    auto issue_b = [&](int kt) {
#pragma unroll
        for (int q = 0; q < B_W; ++q) issue_bq(kt, q);
        const int slot = kt % NSB;
#pragma unroll
        for (int q = 0; q < G::S_W; ++q) {
            const int g = q * NW + wave;
            if (G::NSC % NW == 0 || g < G::NSC)
                dma4(MOE_CHECKED(s_src[q] + scol_bytes(kt), 4, g_scales, g_s_bytes), Ss[slot] + g * 256);
        }
    };

    // W4A4, last stage of a row whose length is not a multiple of 256: each
    // lane zeroes the chunk it loaded if that chunk lies past the row's end
    // (it holds a clamped re-read), so those blocks multiply as zeros.  Runs
    // after the wave's own loads of the stage have landed.
    auto zero_tail = [&](int kt) {
        if (kt * 256 + 4 * lane_col < K) return;
        const int slot = kt % NS;   // NSB == NS here
#pragma unroll
        for (int q = 0; q < A_W; ++q) {
            const int g = q * NW + wave;
            if (g < na_valid) *reinterpret_cast<u32x4 *>(As[slot] + g * 512 + lane * 8) = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < B_W; ++q) {
            const int g = q * NW + wave;
            if (NB % NW == 0 || g < NB)
                *reinterpret_cast<u32x4 *>(Bs[slot] + g * 512 + lane * 8) = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // 4-bit weights straight to LDS, last stage of a row whose length is not
    // a multiple of 256: lanes whose code chunk lies past the row's end zero
    // it (after their own loads of the stage have landed).
    auto zero_tail_w = [&](int kt) {
        if (kt * 256 + 32 * w_ch < K) return;
        const int slot = kt % NSB;
#pragma unroll
        for (int q = 0; q < B_W; ++q) {
            const int g = q * NW + wave;
            if (NB % NW == 0 || g < NB)
                *reinterpret_cast<u32x4 *>(Bs[slot] + g * 512 + lane * 8) = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // ---- MXFP4 weights through registers (one set: committed, then reloaded).
    const char *mb_src[G::MB_PER];
    const uint8_t *ms_src[G::MS_PER];
    u32x4 mb[G::MB_PER];
    uint32_t ms[G::MS_PER][G::SCW];
    if (MX && !WDMA) {
#pragma unroll
        for (int i = 0; i < G::MB_PER; ++i) {
            const int c = (tid + NT * i) % (G::MB_CHUNKS > 0 ? G::MB_CHUNKS : 1);
            const size_t rid = (size_t)e * g_w_rows + weight_row(c / G::CPR);
            mb_src[i] = reinterpret_cast<const char *>(g_w) + rid * (K / 2) + kb / 2 + (c % G::CPR) * 16;
        }
#pragma unroll
        for (int i = 0; i < G::MS_PER; ++i) {
            const int v = (tid + NT * i) % BN;
            ms_src[i] = g_scales + ((size_t)e * g_w_rows + weight_row(v)) * (K / G::SC_BLK) + kb / G::SC_BLK;
        }
    }
    auto issue_mx = [&](int kt) {
#pragma unroll
        for (int i = 0; i < G::MB_PER; ++i)
            mb[i] = *reinterpret_cast<const u32x4 *>(MOE_CHECKED(mb_src[i] + kt * (BK / 2), 16, g_w, g_w_bytes));
        // scale rows are K/32 (E8M0) or K/16 (E4M3) bytes: 2- and 4-byte
        // aligned for K % 64 == 0
#pragma unroll
        for (int i = 0; i < G::MS_PER; ++i)
#pragma unroll
            for (int w = 0; w < G::SCW; ++w) {
                const uint8_t *src = MOE_CHECKED(ms_src[i] + kt * G::SC_PER + 4 * w,
                                                 NV || G::SC_PER >= 4 ? 4 : 2, g_scales, g_s_bytes);
                if (NV) {
                    ms[i][w] = *reinterpret_cast<const uint32_t *>(src);
                } else {
                    const uint32_t lo = *reinterpret_cast<const uint16_t *>(src);
                    ms[i][w] = G::SC_PER >= 4 ? lo | ((uint32_t)*reinterpret_cast<const uint16_t *>(src + 2) << 16)
                                              : lo;
                }
            }
    };
    auto commit_mx = [&](int kt) {
        const int slot = kt % NSB;   // NSB == NS here
        uint32_t *words = reinterpret_cast<uint32_t *>(Bs[slot]);
#pragma unroll
        for (int i = 0; i < G::MB_PER; ++i) {
            const int c = tid + NT * i;
            if (c < G::MB_CHUNKS) {
                const int v = c / G::CPR, part = c % G::CPR;
#pragma unroll
                for (int q = 0; q < 4; ++q) words[(part * 4 + q) * BN + v] = mb[i][q];
            }
        }
#pragma unroll
        for (int i = 0; i < G::MS_PER; ++i) {
            const int v = tid + NT * i;
            if (v < BN) {   // the step's block scales, one byte per block: [block][row]
#pragma unroll
                for (int b = 0; b < G::SC_PER; ++b)
                    Ss[slot][b * BN + v] = (uint8_t)((ms[i][b / 4] >> (8 * (b % 4))) & 0xFFu);
            }
        }
    };

    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int lrow = lane & 15, lk = lane >> 4;

    // ---- W4A4 block scales, staged through LDS one step ahead.  Fragments
    // take a stage's 16-byte chunks in the order ch = 2 lk + kk (any order
    // serves if both operands use it), so a lane's two blocks of a step,
    // 8 kt + 2 lk + kk (kk = 0, 1), are adjacent.  Each thread loads the 8
    // scale bytes of one tile row per step (weight rows first, then token
    // rows) and stores them so that one 32-bit LDS read gives a lane the
    // scales of rows r and r + 16 (bytes 0, 1 and 2, 3; rows in groups of 32
    // aligned to the wave's first row); the MFMA picks its byte itself.  A
    // wave with a single 16-row token tile reads its 16 bits alone.
    const int nblk = K / 32;
    const uint8_t *sc_src = nullptr;   // this thread's scale row
    [[maybe_unused]] const uint8_t *sc_base = nullptr;   // its buffer and extent (bounds checks)
    [[maybe_unused]] size_t sc_bytes = 0;
    int sc_dst = -1;                   // its LDS byte offset (blocks 0, 1 of lane block 0)
    bool sc_pair = true;
    if (A4) {
        if (tid < BN) {
            sc_src = g_scales + ((size_t)e * g_w_rows + weight_row(tid)) * nblk;
            sc_base = g_scales;
            sc_bytes = g_s_bytes;
            sc_dst = ((tid >> 5) * 16 + (tid & 15)) * 16 + ((tid >> 4) & 1) * 2;
        } else if (tid < BN + BM) {
            const int v = tid - BN;
            const int rr = v < rows ? v : 0;
            const size_t src = g_gather ? (size_t)(*MOE_CHECKED(g_gather + seg + rr, 4, g_gather, p.gather_bytes) /
                                                   p.gather_k)
                                        : (size_t)(seg + rr);
            sc_src = p.a_scales + src * nblk;
            sc_base = p.a_scales;
            sc_bytes = p.a_s_bytes;
            sc_pair = G::SC_PAIR_M;
            sc_dst = G::SC_W + (G::SC_PAIR_M ? ((v >> 5) * 16 + (v & 15)) * 16 + ((v >> 4) & 1) * 2 : v * 8);
        }
    }
    uint32_t sc_v[2];   // the step's 8 bytes, in flight between load and store
    // Scale rows of whole 8-byte words (K % 256 == 0, so no partial stage;
    // both scale buffers 8-byte aligned) take one 8-byte load per row and
    // step, others four 2-byte loads: one load instruction of a wave touches
    // up to 64 rows' cache lines, so the narrow form quadruples the requests
    // (measured, W4A4 gate/up at 2048 tokens: 94.1 -> 83.2 us).
    const bool sc_wide = (nblk & 7) == 0 &&
                         ((reinterpret_cast<uintptr_t>(g_scales) | reinterpret_cast<uintptr_t>(p.a_scales)) & 7u) == 0;
    auto load_scales = [&](int kt) {
        if (sc_dst < 0) return;
        if (sc_wide) {
            const uint2 v = *reinterpret_cast<const uint2 *>(MOE_CHECKED(sc_src + 8 * kt, 8, sc_base, sc_bytes));
            sc_v[0] = v.x;
            sc_v[1] = v.y;
            return;
        }
        // blocks past the row (last, partial stage) re-read its last pair;
        // they only scale zeros.  nblk = K/32 is even (K % 64 == 0).
        uint32_t h[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            h[m] = *reinterpret_cast<const uint16_t *>(
                MOE_CHECKED(sc_src + min(8 * kt + 2 * m, nblk - 2), 2, sc_base, sc_bytes));
        sc_v[0] = h[0] | (h[1] << 16);
        sc_v[1] = h[2] | (h[3] << 16);
    };
    auto store_scales = [&](int kt) {
        if (sc_dst < 0) return;
        uint8_t *d = Sc[kt % NS] + sc_dst;
        if (sc_pair) {   // lane block m at bytes 4 m, 4 m + 1 of the pair word
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<uint16_t *>(d + 4 * m) = (uint16_t)(sc_v[m >> 1] >> (16 * (m & 1)));
        } else {
            *reinterpret_cast<uint2 *>(d) = make_uint2(sc_v[0], sc_v[1]);
        }
    };
    // a lane's scale words of weight pair q and token pair q (token tile q
    // alone when unpaired)
    auto read_sw = [&](int slot, int q) -> uint32_t {
        return *reinterpret_cast<const uint32_t *>(Sc[slot] + (((wn * WN) >> 5) + q) * 256 + lrow * 16 + lk * 4);
    };
    auto read_sx = [&](int slot, int q) -> uint32_t {
        if (G::SC_PAIR_M)
            return *reinterpret_cast<const uint32_t *>(Sc[slot] + G::SC_W + (((wm * WTM) >> 5) + q) * 256 +
                                                       lrow * 16 + lk * 4);
        return *reinterpret_cast<const uint16_t *>(Sc[slot] + G::SC_W + (wm * WTM + lrow) * 8 + lk * 2);
    };

    f32x4 acc[NI][MI];
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Router: the fp32 sums of each 256-wide K chunk (256 / BK steps) are
    // added into fp64 in chunk order.
    double acc64[ROUTER ? NI : 1][ROUTER ? MI : 1][4];
    if (ROUTER) {
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc64[j][i][q] = 0.0;
    }
    auto flush = [&]() {
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int i = 0; i < MI; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) acc64[j][i][q] += (double)acc[j][i][q];
                acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
    };

    // A wave whose token rows all lie past the tile's end, or whose weight
    // columns all lie past the last output column, multiplies nothing (its
    // partial tile rows and columns are multiplied anyway: their outputs are
    // simply not stored).
    const bool wave_has_cols = GEGLU ? nt * (BN / 2) + wn * (WN / 2) < g_I : nt * BN + wn * WN < g_n_out;
    const bool wave_mul = wm * WTM < rows && wave_has_cols;   // scalar condition
    // Spread weight loads (deeper weight ring, waves with rows): this wave's
    // B_W weight loads of step kt_b go out one per GAP MFMAs of step kt, so
    // that the loads never stall a wave for long before its MFMAs; they are
    // needed two steps later.
    constexpr bool SPREAD = NSB > NS;
    constexpr int GAP = (KK * MI * NI) / (B_W > 0 ? B_W : 1) > 0 ? (KK * MI * NI) / (B_W > 0 ? B_W : 1) : 1;
    // Operand fragments of MFMA K step kk (32 values) of step kt: weight
    // rows (expanded from 4-bit codes for 4-bit weights) and token rows.
    auto frag_w = [&](int kt, int kk, int j) -> u32x4 {
        const int wslot = kt % NSB;
        const int ch = A4 ? 2 * lk + kk : kk * 4 + lk;
        const int r = wn * WN + j * 16 + lrow;
        if (WDMA) {
            // code row r of the stage: logical chunk kk (32 codes)
            // at physical chunk kk ^ (r & 7) (128-byte rows) or kk ^
            // ((r >> 3) & 1) (32-byte rows); the lane's 8 codes are
            // bytes 4 lk .. 4 lk + 3 of it; scales [row][SC_PER] of
            // the stage, or the tile's [row][SC_ROW] from block SC_PER kt
            const uint8_t *wrow = reinterpret_cast<const uint8_t *>(Bs[wslot]) + r * G::CRB;
            const int pch = G::CCH == 8 ? kk ^ (r & 7) : kk ^ ((r >> 3) & 1);
            const uint32_t codes = *reinterpret_cast<const uint32_t *>(wrow + (pch << 4) + 4 * lk);
            const uint8_t *srow = G::SC_TILE ? Ss[0] + r * G::SC_ROW + G::SC_PER * kt : Ss[wslot] + r * G::SC_PER;
            if (NV) return e2m1x8_times_scale(codes, e4m3_to_f32(srow[2 * kk + (lk >> 1)]));
            const float sc = __uint_as_float((uint32_t)srow[kk] << 23);
            u32x4 v;
            v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
            v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
            v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
            v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
            return v;
        } else if (MX && NV) {
            // E2M1 -> bf16 at scale 1, then times the block's E4M3
            // scale: the product has at most 6 significant bits, so
            // it is exactly a bf16 value (the lane's 8 codes are K
            // 8 ch .. 8 ch + 7, block 2 kk + lk / 2 of the step)
            const uint32_t codes = reinterpret_cast<const uint32_t *>(Bs[wslot])[ch * BN + r];
            const float sc = e4m3_to_f32(Ss[wslot][(2 * kk + (lk >> 1)) * BN + r]);
            return e2m1x8_times_scale(codes, sc);
        } else if (MX) {
            const uint32_t codes = reinterpret_cast<const uint32_t *>(Bs[wslot])[ch * BN + r];
            const float sc = __uint_as_float((uint32_t)Ss[wslot][kk * BN + r] << 23);
            u32x4 v;
            v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
            v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
            v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
            v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
            return v;
        } else {
            return *reinterpret_cast<const u32x4 *>(&Bs[wslot][r * BK + tswz<BK>(r, ch) * 8]);
        }
    };
    auto frag_x = [&](int kt, int kk, int i) -> u32x4 {
        const int ch = A4 ? 2 * lk + kk : kk * 4 + lk;
        const int r = wm * WTM + i * 16 + lrow;
        return *reinterpret_cast<const u32x4 *>(&As[kt % NS][r * BK + tswz<BK>(r, ch) * 8]);
    };
    // The MFMAs of K step kk, with this wave's spread weight loads of step
    // kt_b (if kt_b >= 0) issued among them.
    auto mfma_kk = [&](int kk, const u32x4 *wf, const u32x4 *xf, int kt_b) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                acc[j][i] = mfma16x16x32(wf[j], xf[i], acc[j][i]);
                if constexpr (SPREAD) {
                    const int idx = (kk * MI + i) * NI + j;
                    if (kt_b >= 0 && idx % GAP == GAP - 1 && idx / GAP < B_W) {
                        __builtin_amdgcn_sched_barrier(0);
                        issue_bq(kt_b, idx / GAP);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
    };
    auto compute = [&](int kt, int kt_b) {
        const int slot = kt % NS;
        if constexpr (A4) {
            constexpr int NSW = NI / 2, NSX = G::SC_PAIR_M ? MI / 2 : MI;
            uint32_t sw[NSW], sx[NSX];
#pragma unroll
            for (int q = 0; q < NSW; ++q) sw[q] = read_sw(slot, q);
#pragma unroll
            for (int q = 0; q < NSX; ++q) sx[q] = read_sx(slot, q);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                u32x4 wf[NI], xf[MI];
#pragma unroll
                for (int j = 0; j < NI; ++j) wf[j] = frag_w(kt, kk, j);
#pragma unroll
                for (int i = 0; i < MI; ++i) xf[i] = frag_x(kt, kk, i);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        acc[j][i] = mfma_fp4x128(wf[j], xf[i], acc[j][i], sw[j / 2], sx[G::SC_PAIR_M ? i / 2 : i],
                                                 2 * (j & 1) + kk, (G::SC_PAIR_M ? 2 * (i & 1) : 0) + kk);
            }
        } else {
            // Per MFMA K step of 32: the fragments, then the MFMAs.
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                u32x4 wf[NI], xf[MI];
#pragma unroll
                for (int j = 0; j < NI; ++j) wf[j] = frag_w(kt, kk, j);
#pragma unroll
                for (int i = 0; i < MI; ++i) xf[i] = frag_x(kt, kk, i);
                mfma_kk(kk, wf, xf, kt_b);
            }
        }
    };

    // ---- pipeline.  Step kt: wait until its loads have landed (loads of
    // later steps already issued may stay in flight), publish, issue the
    // token tile of step kt + NS - 1 and the weight tile of step kt + NSB - 1
    // into the stages freed by step kt - 1, then multiply.  The issue order
    // (below, at wait_for) keeps the counts exact.
    // Loads this wave issues per step: its valid token-row groups and its
    // weight-row groups (exact, so each wave waits for no more than it must).
    int dma_per_step = 0;
#pragma unroll
    for (int q = 0; q < A_W; ++q) dma_per_step += (q * NW + wave < na_valid) ? 1 : 0;
#pragma unroll
    for (int q = 0; q < B_W; ++q) dma_per_step += b_on[q] ? 1 : 0;
#pragma unroll
    for (int q = 0; q < G::S_W; ++q) dma_per_step += (G::NSC % NW == 0 || q * NW + wave < G::NSC) ? 1 : 0;
    // This wave's weight (and scale) loads per step.
    int dmab_per_step = 0;
#pragma unroll
    for (int q = 0; q < B_W; ++q) dmab_per_step += b_on[q] ? 1 : 0;
#pragma unroll
    for (int q = 0; q < G::S_W; ++q) dmab_per_step += (G::NSC % NW == 0 || q * NW + wave < G::NSC) ? 1 : 0;
    // Issue order: the prologue issues, for s = 0, 1, ..., the token tile of
    // step s (s < NS - 1) and then the weight tile of step s (s < NSB - 1);
    // step kt issues the token tile of kt + NS - 1, then the weight tile of
    // kt + NSB - 1.  At the top of step kt the loads issued after the last
    // one it needs are: NSB == NS: the NS - 2 later steps' loads; NS = 2,
    // NSB > 2: the weight tile of kt + NSB - 2, issued (in step kt - 1)
    // right after the token tile of kt.  (In step 0 this waits for more than
    // it needs: the prologue's later weight tiles.)
    auto wait_for = [&](int kt) {
        if constexpr (NSB == NS) {
            const int later = min(NS - 2, KT - 1 - kt);   // steps issued after kt
            wait_vm_lgkm0_rt(later * dma_per_step);
        } else {
            wait_vm_lgkm0_rt(kt + NSB - 2 < KT ? dmab_per_step : 0);
        }
    };
    // Output rows of this lane's token rows when the output is scattered
    // (loaded before the first loads of the pipeline, so that they are older
    // than every load its wait counts cover).
    const bool out_map = MODE == kDown && !shared && p.out_rows != nullptr;
    int out_row[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int t = wm * WTM + i * 16 + lrow;
        out_row[i] = out_map && t < rows ? *MOE_CHECKED(p.out_rows + seg + t, 4, p.out_rows, p.out_rows_bytes) : 0;
    }
    if (MX && !WDMA) issue_mx(0);
    if (A4) {
        load_scales(0);
        store_scales(0);   // published by the first step's barrier
    }
#pragma unroll
    for (int s0 = 0; s0 < NSB - 1; ++s0) {
        if (s0 < NS - 1 && s0 < KT) issue_a(s0);
        if (s0 < KT) issue_b(s0);
    }
    // Per-tile block scales (4-bit codes straight to LDS in 64-wide steps):
    // the tile's whole scale rows, K/32 bytes each, read into LDS once,
    // NT/BN threads per row, in 16-bit words.  They are issued after the
    // first stages' loads so that the latencies overlap; the compiler's own
    // wait before the LDS stores then also covers those stages, which the
    // first step waits for anyway, so the pipeline's counts stay exact.
    if constexpr (G::SC_TILE) {
        constexpr int TPR = NT / BN, MAXW = (G::SC_ROW / 2 + TPR - 1) / TPR;
        static_assert(NT % BN == 0, "whole threads per scale row");
        const int v = tid % BN, w0 = tid / BN, nh = K / (2 * G::SC_BLK);   // 16-bit words per scale row
        const uint16_t *srow = reinterpret_cast<const uint16_t *>(
            g_scales + ((size_t)e * g_w_rows + weight_row(v)) * (size_t)(K / G::SC_BLK));
        uint16_t sv[MAXW];
#pragma unroll
        for (int i = 0; i < MAXW; ++i)
            if (TPR * i < nh) sv[i] = *MOE_CHECKED(srow + min(w0 + TPR * i, nh - 1), 2, g_scales, g_s_bytes);
        uint16_t *dst = reinterpret_cast<uint16_t *>(Ss[0] + v * G::SC_ROW);
#pragma unroll
        for (int i = 0; i < MAXW; ++i)
            if (w0 + TPR * i < nh) dst[w0 + TPR * i] = sv[i];
    }
    // The loop is instantiated twice so that the accumulators are never live
    // across a branch: waves with rows multiply, the others only load.
    auto run = [&](auto mul_c) {
        constexpr bool MUL = decltype(mul_c)::value;
        for (int kt = 0; kt < KT; ++kt) {
            wait_for(kt);
            if (A4 && kt == KT - 1 && (K & 255)) {
                zero_tail(kt);
                wait_vm_lgkm0<63>();      // the zeroes are in LDS
            }
            if (WDMA && BK == 256 && kt == KT - 1 && (K & 255)) {
                zero_tail_w(kt);
                wait_vm_lgkm0<63>();
            }
            if (MX && !WDMA) {
                commit_mx(kt);
                wait_vm_lgkm0<63>();      // this wave's LDS writes are done
            }
            __builtin_amdgcn_s_barrier();
            if (MX && !WDMA && kt + 1 < KT) issue_mx(kt + 1);
            // scales of step kt + 1: loaded before the DMA (so in-order
            // counts cover them), stored after this step's MFMAs are issued
            const bool next_sc = A4 && kt + 1 < KT;
            if (next_sc) load_scales(kt + 1);
            if (kt + NS - 1 < KT) issue_a(kt + NS - 1);
            const bool spread = SPREAD && MUL && kt + NSB - 1 < KT;
            if (kt + NSB - 1 < KT && !spread) issue_b(kt + NSB - 1);
            if (MUL) {
                compute(kt, spread ? kt + NSB - 1 : -1);
                if (ROUTER && ((kt % (256 / BK)) == 256 / BK - 1 || kt == KT - 1)) flush();
            }
            if (next_sc) {
                // keep the store (and the wait for its loads that comes with
                // it) behind the MFMAs
                __builtin_amdgcn_sched_barrier(0);
                store_scales(kt + 1);
            }
        }
    };
    if (wave_mul) run(std::true_type{});
    else run(std::false_type{});

    // ---- epilogue: lane holds weight rows 4*lk .. 4*lk+3 of tile j for the
    // token lrow of token tile i.  NVFP4: the expert matrix's fp32 scale
    // (times the activations' input scale for NVFP4 activations) multiplies
    // the fp32 sums (before the GEGLU).
    const float gsc = NV ? p.w_global[e] * (p.a_global ? *p.a_global : 1.0f) : 1.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int t = wm * WTM + i * 16 + lrow;
        if (t >= rows) continue;
        uint16_t *orow = g_out + (size_t)(out_map ? out_row[i] : seg + t) * g_n_out;
        if (ROUTER) {
            float *lrow_out = p.out32 + (size_t)(seg + t) * p.n_out;
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = nt * BN + wn * WN + j * 16 + 4 * lk + q;
                    if (n < p.n_out) {
                        const double b = p.bias ? (double)p.bias[n] : 0.0;
                        *MOE_CHECKED(lrow_out + n, 4, p.out32, p.out_bytes) = (float)(acc64[j][i][q] + b);
                    }
                }
        } else if (GEGLU && (NI / 2) % 2 == 0) {
            // pairs of adjacent 16-column fragments: lanes l and l ^ 16 (k
            // groups lk and lk ^ 1) swap half their values so that each lane
            // stores 8 consecutive bf16 (16 bytes) and a row gets 64
            // contiguous bytes per store instruction
            constexpr int HALF_T = NI / 2;
#pragma unroll
            for (int j = 0; j < HALF_T; j += 2) {
                const int n0 = nt * (BN / 2) + wn * (WN / 2) + j * 16;
                uint2 p[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    f32x4 g = acc[j + d][i], u = acc[j + d + HALF_T][i];
                    if (NV) {
                        g *= gsc;
                        u *= gsc;
                    }
                    p[d].x = pack_bf16x2(gelu_tanh(g[0]) * u[0], gelu_tanh(g[1]) * u[1]);
                    p[d].y = pack_bf16x2(gelu_tanh(g[2]) * u[2], gelu_tanh(g[3]) * u[3]);
                }
                const int odd = lk & 1;
                const uint4 o = pair_swap16(p[0], p[1], odd);
                const int n = n0 + odd * 16 + 4 * (lk & ~1);
                if (n < g_I) *reinterpret_cast<uint4 *>(MOE_CHECKED(orow + n, 16, g_out, g_out_bytes)) = o;
            }
        } else if (GEGLU) {
            constexpr int HALF_T = NI / 2;
#pragma unroll
            for (int j = 0; j < HALF_T; ++j) {
                const int n = nt * (BN / 2) + wn * (WN / 2) + j * 16 + 4 * lk;
                if (n >= g_I) continue;
                f32x4 g = acc[j][i], u = acc[j + HALF_T][i];
                if (NV) {
                    g *= gsc;
                    u *= gsc;
                }
                uint2 o;
                o.x = pack_bf16x2(gelu_tanh(g[0]) * u[0], gelu_tanh(g[1]) * u[1]);
                o.y = pack_bf16x2(gelu_tanh(g[2]) * u[2], gelu_tanh(g[3]) * u[3]);
                *reinterpret_cast<uint2 *>(MOE_CHECKED(orow + n, 8, g_out, g_out_bytes)) = o;
            }
        } else if (shared && p.sh_out32) {   // dense MLP down: fp32 partial sum of this K range
            float *prow = p.sh_out32 + ((size_t)split * p.sh_rows + seg + t) * g_n_out;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int n = nt * BN + wn * WN + j * 16 + 4 * lk;
                if (n >= g_n_out) continue;
                *reinterpret_cast<f32x4 *>(MOE_CHECKED(prow + n, 16, p.sh_out32, p.sh_out_bytes)) = acc[j][i];
            }
        } else if (NI % 2 == 0) {
#pragma unroll
            for (int j = 0; j < NI; j += 2) {   // fragment pairs, 16 bytes per lane (as above)
                uint2 pr[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    f32x4 v = acc[j + d][i];
                    if (NV) v *= gsc;
                    pr[d].x = pack_bf16x2(v[0], v[1]);
                    pr[d].y = pack_bf16x2(v[2], v[3]);
                }
                const int odd = lk & 1;
                const uint4 o = pair_swap16(pr[0], pr[1], odd);
                const int n = nt * BN + wn * WN + (j + odd) * 16 + 4 * (lk & ~1);
                if (n < g_n_out) *reinterpret_cast<uint4 *>(MOE_CHECKED(orow + n, 16, g_out, g_out_bytes)) = o;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int n = nt * BN + wn * WN + j * 16 + 4 * lk;
                if (n >= g_n_out) continue;
                f32x4 v = acc[j][i];
                if (NV) v *= gsc;
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2 *>(MOE_CHECKED(orow + n, 8, g_out, g_out_bytes)) = o;
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

template <int BM, int BN, int WM, int WN, int MODE, bool MX, int NS, int BK, bool A4 = false, bool NV = false,
          bool WD = false, int NSB = 0>
static hipError_t launch_cfg(GemmArgs a, int A, hipStream_t st) {
    constexpr bool GEGLU = MODE == kGateUp;
    const int ncols = GEGLU ? a.I : a.n_out;
    const int per_tile = GEGLU ? BN / 2 : BN;
    a.n_tiles = (ncols + per_tile - 1) / per_tile;
    // An expert whose rows fit one row tile is the only reader of its weight
    // slab, so its loads carry the streaming hint.  When the mean expert has
    // more than BM/2 rows, most slabs are re-read by several row tiles, and
    // streaming the few single-tile experts was measured to slow the launch
    // (Zipf-skewed prefill of 8192 tokens: 1.6%), so none stream then.
    a.stream_max_rows = (MODE != kRouter && !MX && A / a.E <= BM / 2) ? BM : 0;
    const int slots = MODE == kRouter ? (a.dense_rows + BM - 1) / BM : mtile_slots(A, a.E, BM);
    // whole rounds of 8 groups (one per XCD)
    long long blocks = (long long)a.n_tiles * ((slots + 7) / 8 * 8);
    a.routed_blocks = (int)blocks;
    // every group's K must be whole steps (the kernel loops K / BK times)
    // (W4A4 and 4-bit weights in 256-wide steps end with a partial stage)
    constexpr bool PARTIAL = A4 || (MX && BK == 256);
    if (PARTIAL ? (a.K % 64 != 0 || a.sh_rows > 0)
                : (a.K % BK != 0 || (MODE != kRouter && a.sh_rows > 0 && (a.sh_K % BK != 0 || a.sh_ksplit % BK != 0))))
        return hipErrorInvalidValue;
    if (MODE != kRouter && a.sh_rows > 0) {
        a.sh_n_tiles = GEGLU ? (a.sh_I + BN / 2 - 1) / (BN / 2) : (a.sh_n_out + BN - 1) / BN;
        blocks += (long long)a.sh_n_tiles * ((a.sh_rows + BM - 1) / BM) * max(1, a.sh_splits);
    }
    if (blocks == 0) return hipSuccess;
    grouped_gemm_kernel<BM, BN, WM, WN, MODE, MX, NS, BK, A4, NV, WD, NSB>
        <<<dim3((unsigned)blocks), 64 * WM * WN, 0, st>>>(a);
    return hipGetLastError();
}

// Row-block size from the mean rows per expert (a function of the shape
// only, so the launch does not depend on the routing).
template <int MODE, bool MX, bool NV = false>
static hipError_t launch_sized(const GemmArgs &a, int A, hipStream_t st) {
    const int mean_rows = A / a.E;
    // Small row blocks stream weights: two stages keep LDS small enough for
    // four workgroups per CU.  The 256 x 256 block runs one workgroup of
    // sixteen waves (4 x 4, 64 tokens x 64 weight rows each) per CU: the
    // large tile moves the fewest bytes per FLOP through the per-CU load
    // path, and at <= 128 rows per expert (the first two token groups busy)
    // each SIMD still has two multiplying waves, so one wave's LDS reads and
    // waits overlap another's MFMAs (eight waves, 4 x 2, left one per SIMD:
    // measured at 2048 tokens, gate/up 239 -> 220 us bf16 and 228 -> 194 us
    // MXFP4).  bf16 with two token and three weight stages (the 160 KB of
    // LDS), MXFP4 (small weight tiles) in three stages of both.  (Measured:
    // K steps of 32 in four stages are slower.)
    if (mean_rows <= 16) {
        // bf16 weight rows are read in 256-byte pieces per step where K
        // allows it (measured: 2% faster than 128-byte pieces at 2816 x
        // 1408).  Not with a shared group: its K need not be a multiple of
        // 128, and the smaller stages keep four workgroups per CU, so routed
        // and shared tiles run in one round.  4-bit weights take 256 K values
        // per step where K allows it: code rows in 128-byte pieces and their
        // scales go straight to LDS in three stages (two steps in flight;
        // the register route of 64-wide steps has one step of 32 bytes per
        // row in flight).
        if constexpr (!MX) {
            if (a.K % 128 == 0 && a.sh_rows == 0) return launch_cfg<16, 128, 1, 4, MODE, MX, 2, 128>(a, A, st);
        } else {
            // codes 16-byte and scale rows 4-byte aligned for the direct
            // loads (any K % 64 == 0: a partial last stage is handled).
            // Rows shorter than 1024 keep the register route: three or fewer
            // steps never fill the three stages, and the 80 KB of LDS halves
            // the workgroups per CU (measured, NVFP4 down at K = 704: 30.1
            // against 24.6 us).
            const bool aligned = (reinterpret_cast<uintptr_t>(a.w) & 15u) == 0 &&
                                 (reinterpret_cast<uintptr_t>(a.scales) & 3u) == 0 && (a.K / (NV ? 16 : 32)) % 4 == 0;
            if (a.sh_rows == 0 && aligned && a.K >= 1024)
                return launch_cfg<16, 128, 1, 4, MODE, MX, 3, 256, false, NV>(a, A, st);
        }
        // With the shared group (three K ranges x 22 column tiles of the
        // dense MLP's down) the 128-column down tiles of a decode step
        // outnumber the 1024 slots of four workgroups per CU, and the last
        // ones run alone; 192-column tiles (three per CU) fit one round
        // (measured, 8 tokens with the 2112-wide MLP: step 116.5 -> 111.6
        // us, down 41.0 -> 36.3 us; without the MLP no change).
        if constexpr (MODE == kDown && !MX)
            if (a.sh_rows > 0) return launch_cfg<16, 192, 1, 4, MODE, MX, 2, 64, false, NV>(a, A, st);
        return launch_cfg<16, 128, 1, 4, MODE, MX, 2, 64, false, NV>(a, A, st);
    }
    // Above 16: the row tile holds a typical expert's rows whole (mean plus
    // a few standard deviations), so each weight slab is streamed once
    // rather than once per row tile: 64-row tiles up to a mean of 40 rows,
    // the 256 x 256 tile above (measured: 512 tokens, 64- instead of 32-row
    // tiles, step 376 -> 295 us; 1024 tokens, 256- instead of 64-row tiles,
    // 398 -> 336 us).
    if (mean_rows <= 40) return launch_cfg<64, 128, 2, 2, MODE, MX, 2, 64, false, NV>(a, A, st);
    if constexpr (MX) {
        // 4-bit codes straight to LDS (16-byte aligned rows of K/2 bytes)
        // with the tile's scale rows (K/32 E8M0 or K/16 E4M3 bytes, 2-byte
        // aligned, at most SC_ROW) read into LDS once: no register staging in
        // the K loop (NVFP4 weights and activations at 2048 tokens: layer step
        // 625 -> 521 us, gate/up 368 -> 289 us, down 198 -> 165 us against
        // the register route in eight waves).
        // Waves 4 x 4: each weight fragment is expanded by four waves, but
        // two waves per SIMD multiply at <= 128 rows (2 x 8 waves, two
        // expansions per fragment: 217 us; 4 x 4: 194 us for the gate/up at
        // 2048 tokens).  Two token stages and a deeper ring of code stages
        // (8 KB each): six for gate/up (K = 2816: 44 steps), four for down
        // (K = 704: 11 steps, where a long prologue costs more than it
        // hides).  Measured at 2048 tokens against three + three stages:
        // gate/up 201 -> 187 us (six) and 192 us (four), down 122.5 ->
        // 120.4 us (four) and 125.5 us (six).
        constexpr int NSB = MODE == kGateUp ? 6 : 4;
        using Tile = GemmTile<256, 256, 4, 4, MODE, MX, 2, 64, false, NV, true, NSB>;
        const bool direct = (reinterpret_cast<uintptr_t>(a.w) & 15u) == 0 &&
                            (reinterpret_cast<uintptr_t>(a.scales) & 1u) == 0 && a.K >= 128 &&
                            a.K / Tile::SC_BLK <= Tile::SC_ROW;
        if (direct && a.sh_rows == 0)
            return launch_cfg<256, 256, 4, 4, MODE, MX, 2, 64, false, NV, true, NSB>(a, A, st);
    }
    if constexpr (!MX)
        return launch_cfg<256, 256, 4, 4, MODE, MX, 2, 64, false, NV, false, 3>(a, A, st);
    else
        return launch_cfg<256, 256, 4, 2, MODE, MX, 3, 64, false, NV>(a, A, st);
}

// W4A4: K steps of 256 codes, and the row-block rule of the bf16 tiles (a
// typical expert's rows in one row tile, so its weights stream once): 16
// rows up to a mean of 16 rows per expert, 64 up to 40, 256 above
// (measured, layer step: 512 tokens 180.0 -> 155.4 us against 32-row tiles,
// 1024 tokens 208.5 -> 193.2 us against 64-row tiles).
template <int MODE>
static hipError_t launch_sized_a4(const GemmArgs &a, int A, hipStream_t st) {
    const int mean_rows = A / a.E;
    if (mean_rows <= 16) return launch_cfg<16, 128, 1, 4, MODE, false, 2, 64, true>(a, A, st);
    if (mean_rows <= 40) return launch_cfg<64, 128, 2, 2, MODE, false, 2, 64, true>(a, A, st);
    return launch_cfg<256, 256, 4, 4, MODE, false, 2, 64, true>(a, A, st);
}

hipError_t launch_gateup_a4(const uint8_t *xq, const uint8_t *xs, const int32_t *sorted_ids, int k,
                            const int32_t *offsets, const void *w, const uint8_t *scales, uint16_t *h, int A, int H,
                            int E, int I, hipStream_t st) {
    GemmArgs a{reinterpret_cast<const uint16_t *>(xq), sorted_ids, k, offsets, w, scales, h, E, H, I, I, 2 * I,
               0, 0, 0, nullptr, nullptr};
    a.a_scales = xs;
    const size_t T = (size_t)A / k;
    a.a_bytes = T * H / 2;
    a.a_s_bytes = T * H / 32;
    a.gather_bytes = (size_t)A * 4;
    a.w_bytes = (size_t)E * 2 * I * H / 2;
    a.s_bytes = (size_t)E * 2 * I * H / 32;
    a.out_bytes = (size_t)A * I * 2;
    return launch_sized_a4<kGateUp>(a, A, st);
}

// The combine reads the down GEMM's output y right after it.  When y is
// larger than the last-level cache (256 MB on MI355X) the down GEMM runs its
// row-tile groups last to first, which leaves more of the rows the combine
// reads in that cache (measured, 8192 Zipf-skewed tokens, y = 369 MB: down
// 376 -> 358 us, combine 78 -> 64 us); when y fits, the forward order is
// faster (2048 tokens: down 131 against 136 us).
constexpr long long kLastLevelCacheBytes = 256LL << 20;
static int reverse_down_groups(int A, int H) { return (long long)A * H * 2 > kLastLevelCacheBytes ? 1 : 0; }

hipError_t launch_down_a4(const uint8_t *hq, const uint8_t *hs, const int32_t *offsets, const void *w,
                          const uint8_t *scales, uint16_t *y, const int32_t *out_rows, int A, int H, int E, int I,
                          hipStream_t st) {
    GemmArgs a{reinterpret_cast<const uint16_t *>(hq), nullptr, 1, offsets, w, scales, y, E, I, H, I, H, 0, 0, 0,
               nullptr, nullptr};
    a.out_rows = out_rows;
    a.out_rows_bytes = (size_t)A * 4;
    a.a_scales = hs;
    a.a_bytes = (size_t)A * I / 2;
    a.a_s_bytes = (size_t)A * I / 32;
    a.w_bytes = (size_t)E * H * I / 2;
    a.s_bytes = (size_t)E * H * I / 32;
    a.out_bytes = (size_t)A * H * 2;
    a.reverse_groups = reverse_down_groups(A, H);
    return launch_sized_a4<kDown>(a, A, st);
}

hipError_t launch_gateup(const uint16_t *x, const int32_t *sorted_ids, int k, const int32_t *offsets,
                         const void *w, const uint8_t *scales, const float *w_global, const float *a_global,
                         uint16_t *h, int A, int H, int E, int I, WeightFormat fmt, const SharedGroup *sh,
                         hipStream_t st) {
    GemmArgs a{x, sorted_ids, k, offsets, w, scales, h, E, H, I, I, 2 * I, 0, 0, 0, nullptr, nullptr};
    a.w_global = w_global;
    a.a_global = a_global;
    // extents (bounds checks): x gathered from [T][H] or pre-permuted [A][H];
    // weights [E][2I][H] bf16 or 4-bit codes; block scales per 32 or 16
    const size_t wk = fmt == WeightFormat::kBF16 ? 2 * (size_t)H : (size_t)H / 2;
    const size_t sk = fmt == WeightFormat::kMXFP4 ? H / 32 : (fmt == WeightFormat::kNVFP4 ? H / 16 : 0);
    a.a_bytes = (sorted_ids ? (size_t)A / k : (size_t)A) * H * 2;
    a.gather_bytes = (size_t)A * 4;
    a.w_bytes = (size_t)E * 2 * I * wk;
    a.s_bytes = (size_t)E * 2 * I * sk;
    a.out_bytes = (size_t)A * I * 2;
    if (sh) {   // every token through the shared gate/up weights [2 I_sh][H]
        a.sh_rows = sh->rows;
        a.sh_a = x;
        a.sh_w = sh->w;
        a.sh_scales = sh->scales;
        a.sh_out = sh->out;
        a.sh_K = H;
        a.sh_I = sh->I;
        a.sh_w_rows = 2 * sh->I;
        a.sh_n_out = sh->I;
        a.sh_splits = 1;
        a.sh_ksplit = H;
        a.sh_a_bytes = (size_t)sh->rows * H * 2;
        a.sh_w_bytes = 2 * (size_t)sh->I * wk;
        a.sh_s_bytes = 2 * (size_t)sh->I * sk;
        a.sh_out_bytes = (size_t)sh->rows * sh->I * 2;
    }
    if (fmt == WeightFormat::kNVFP4) return sh ? hipErrorInvalidValue : launch_sized<kGateUp, true, true>(a, A, st);
    return fmt == WeightFormat::kMXFP4 ? launch_sized<kGateUp, true>(a, A, st) : launch_sized<kGateUp, false>(a, A, st);
}

hipError_t launch_down(const uint16_t *h, const int32_t *offsets, const void *w, const uint8_t *scales,
                       const float *w_global, const float *a_global, uint16_t *y, const int32_t *out_rows, int A,
                       int H, int E, int I, WeightFormat fmt, const SharedGroup *sh, hipStream_t st) {
    GemmArgs a{h, nullptr, 1, offsets, w, scales, y, E, I, H, I, H, 0, 0, 0, nullptr, nullptr};
    a.out_rows = out_rows;
    a.out_rows_bytes = (size_t)A * 4;
    a.w_global = w_global;
    a.a_global = a_global;
    a.reverse_groups = reverse_down_groups(A, H);
    // extents (bounds checks): h [A][I]; weights [E][H][I] bf16 or 4-bit
    // codes; block scales per 32 or 16
    const size_t wk = fmt == WeightFormat::kBF16 ? 2 * (size_t)I : (size_t)I / 2;
    const size_t sk = fmt == WeightFormat::kMXFP4 ? I / 32 : (fmt == WeightFormat::kNVFP4 ? I / 16 : 0);
    a.a_bytes = (size_t)A * I * 2;
    a.w_bytes = (size_t)E * H * wk;
    a.s_bytes = (size_t)E * H * sk;
    a.out_bytes = (size_t)A * H * 2;
    if (sh) {   // the shared h rows [rows][I_sh] through the shared down weights [H][I_sh]
        a.sh_rows = sh->rows;
        a.sh_a = sh->a;
        a.sh_w = sh->w;
        a.sh_scales = sh->scales;
        a.sh_out = sh->out;
        a.sh_out = nullptr;
        a.sh_out32 = sh->out32;
        a.sh_K = sh->I;
        a.sh_I = sh->I;
        a.sh_w_rows = H;
        a.sh_n_out = H;
        // K cut into ranges about as long as an expert's (I), so a shared
        // tile takes as long as a routed one; partial sums stay fp32
        a.sh_splits = shared_splits(sh->I, I);
        a.sh_ksplit = shared_ksplit(sh->I, I);
        const size_t swk = fmt == WeightFormat::kBF16 ? 2 * (size_t)sh->I : (size_t)sh->I / 2;
        a.sh_a_bytes = (size_t)sh->rows * sh->I * 2;
        a.sh_w_bytes = (size_t)H * swk;
        a.sh_s_bytes = fmt == WeightFormat::kMXFP4 ? (size_t)H * sh->I / 32 : 0;
        a.sh_out_bytes = (size_t)a.sh_splits * sh->rows * H * 4;
    }
    if (fmt == WeightFormat::kNVFP4) return sh ? hipErrorInvalidValue : launch_sized<kDown, true, true>(a, A, st);
    return fmt == WeightFormat::kMXFP4 ? launch_sized<kDown, true>(a, A, st) : launch_sized<kDown, false>(a, A, st);
}

// Router for many tokens: x [T][H] times W_r [E][H]^T as one dense group, 16
// tokens x 64 experts per workgroup; K steps as long as H allows (fewer
// steps of a latency-bound loop: 64 -> 128 measured 23 -> 18.5 us for the
// routing at 2048 tokens, 128 in four stages -> 256 in three 18.5 -> 17.5
// us; a step of 256 is one chunk of the logit definition).  From 8192
// tokens (256 tiles of 32 tokens) the tile is 32
// tokens x 128 experts in three stages: half the operand bytes per FLOP
// through the per-CU load path (8192 tokens: 43.6 -> 35.6 us for the
// routing; at 2048 tokens, 64 such tiles leave most CUs idle: 18 -> 29 us),
// in eight waves of 16 tokens x 32 experts (four waves: 37.0 us for the
// routing at 8192 tokens, eight: 31.1 us).
hipError_t launch_router_dense(const uint16_t *x, const uint16_t *wr, const float *bias, float *logits,
                               int T, int H, int E, hipStream_t st) {
    GemmArgs a{x, nullptr, 1, nullptr, wr, nullptr, nullptr, 1, H, E, 0, E, 0, 0, T, logits, bias};
    a.a_bytes = (size_t)T * H * 2;
    a.w_bytes = (size_t)E * H * 2;
    a.out_bytes = (size_t)T * E * 4;
    if (H % 128 == 0 && T >= 8192) return launch_cfg<32, 128, 2, 4, kRouter, false, 3, 128>(a, T, st);
    if (H % 256 == 0) return launch_cfg<16, 64, 1, 4, kRouter, false, 3, 256>(a, T, st);
    if (H % 128 == 0) return launch_cfg<16, 64, 1, 4, kRouter, false, 4, 128>(a, T, st);
    return launch_cfg<16, 64, 1, 4, kRouter, false, 6, 64>(a, T, st);
}

#ifdef MOE_DEBUG
MOE_DEBUG_READER(debug_read_gemm)
#endif

}  // namespace moe
