// Internal launchers of the MoE kernels (host side, called by the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kChunk = 1024;           // assignments per permutation block
constexpr int kSmallRouteMaxA = 2048;  // fused few-token top-k + permutation: T*k up to this

constexpr int kRouterSplitMaxT = 64;   // split-K router (chunk partials) up to this many tokens
constexpr int kFusedRouteMaxT = 16;    // single-launch routing up to this many tokens (one per wave)

int router_chunks(int H);
bool router_uses_partials(int T);
// Few tokens: fp32 chunk sums part[router_chunks(H)][T][E].
hipError_t launch_router_partials(const uint16_t *x, const uint16_t *wr, float *part, int T, int H, int E,
                                  hipStream_t st);
// Many tokens: final fp32 logits [T][E] from the grouped GEMM engine.
hipError_t launch_router_dense(const uint16_t *x, const uint16_t *wr, const float *bias, float *logits,
                               int T, int H, int E, hipStream_t st);
// Top-k from chunk partials (part != nullptr; logits optional output) or
// from final logits (part == nullptr).
hipError_t launch_topk(const float *part, int nchunks, const float *bias, float *logits, int32_t *ids,
                       float *w, int T, int E, int k, hipStream_t st);
// Few tokens (route_permute_fits: T <= kFusedRouteMaxT): router chunk sums,
// top-k and the whole permutation (counts, offsets, sorted_ids, inv) in one
// launch.  `done` is a
// completion counter that must be zero before the launch; it is zero again
// after it.
bool route_permute_fits(int T, int k);
hipError_t launch_route_permute(const uint16_t *x, const uint16_t *wr, float *part, uint32_t *done,
                                const float *bias, float *logits, int32_t *ids, float *w, int32_t *counts,
                                int32_t *offsets, int32_t *sorted_ids, int32_t *inv, int T, int H, int E, int k,
                                hipStream_t st);
hipError_t launch_permute(const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_ids, int32_t *inv, int32_t *block_hist, int A, int E,
                          hipStream_t st);
hipError_t launch_gather_rows(const uint16_t *x, const int32_t *sorted_ids, uint16_t *x_perm,
                              int A, int H, int k, hipStream_t st);
// Optional always-on group of the grouped GEMMs: a dense GEGLU MLP applied
// to every token (a shared expert), tiled in the same launch as the routed
// experts.  Gate/up: a = x (unused field), w = [2 I][H], out = h_sh
// [rows][I] bf16; down: a = h_sh, w = [H][I], out32 = fp32 partial sums
// [shared_splits(I, I_expert)][rows][H] over consecutive K ranges.
struct SharedGroup {
    const uint16_t *a;
    const void *w;
    const uint8_t *scales;   // MXFP4 scales or nullptr
    uint16_t *out;
    float *out32;
    int rows, I;
};
// K ranges of the dense MLP's down GEMM: about I_sh / I_expert of them, each
// a whole number of 64-wide steps, none empty (the last may be shorter).
inline int shared_ksplit(int I_sh, int I_expert) {
    int n = (I_sh + I_expert / 2) / I_expert;
    if (n < 1) n = 1;
    const int units = I_sh / 64;
    return 64 * ((units + n - 1) / n);
}
inline int shared_splits(int I_sh, int I_expert) {
    const int ks = shared_ksplit(I_sh, I_expert);
    return (I_sh + ks - 1) / ks;
}
// Expert weight formats of the grouped GEMMs: bf16; MXFP4 (scales: E8M0
// [E][rows][K/32]); NVFP4 (scales: E4M3 [E][rows][K/16], w_global: the fp32
// scale of each expert's matrix [E]; no shared group).
// a_global (NVFP4 only, or nullptr): the fp32 input scale of activations
// that arrive decoded without it (NVFP4 activations), applied with w_global.
enum class WeightFormat { kBF16, kMXFP4, kNVFP4 };
hipError_t launch_gateup(const uint16_t *x, const int32_t *sorted_ids, int k, const int32_t *offsets,
                         const void *w, const uint8_t *scales, const float *w_global, const float *a_global,
                         uint16_t *h, int A, int H, int E, int I, WeightFormat fmt, const SharedGroup *sh,
                         hipStream_t st);
// out_rows (or nullptr): grouped row r of y goes to row out_rows[r] (the
// layer passes sorted_ids, which puts y in (token, slot) order).
hipError_t launch_down(const uint16_t *h, const int32_t *offsets, const void *w, const uint8_t *scales,
                       const float *w_global, const float *a_global, uint16_t *y, const int32_t *out_rows, int A,
                       int H, int E, int I, WeightFormat fmt, const SharedGroup *sh, hipStream_t st);
// W4A4 grouped GEMMs: activations as MXFP4 codes [rows][K/2] + E8M0 scales
// [rows][K/32] (launch_quantize_mx), weights MXFP4; K a multiple of 64.
hipError_t launch_gateup_a4(const uint8_t *xq, const uint8_t *xs, const int32_t *sorted_ids, int k,
                            const int32_t *offsets, const void *w, const uint8_t *scales, uint16_t *h, int A, int H,
                            int E, int I, hipStream_t st);
hipError_t launch_down_a4(const uint8_t *hq, const uint8_t *hs, const int32_t *offsets, const void *w,
                          const uint8_t *scales, uint16_t *y, const int32_t *out_rows, int A, int H, int E, int I,
                          hipStream_t st);
// MXFP4 codes and scales of bf16 rows [rows][K], K a multiple of 32.
hipError_t launch_quantize_mx(const uint16_t *src, long long rows, int K, uint8_t *codes, uint8_t *scales,
                              hipStream_t st);
// NVFP4 quantisation of bf16 rows [rows][K] (K a multiple of 16) relative
// to the fp32 input scale *g: codes [rows][K/2] and E4M3 scales [rows][K/16]
// (both or neither), and/or the decoded values without g as bf16 into dq
// [rows][K] (dq may be src itself).
hipError_t launch_quantize_nv(const uint16_t *src, long long rows, int K, const float *g, uint8_t *codes,
                              uint8_t *scales, uint16_t *dq, hipStream_t st);
// y_sh32 (optional, [nsplit][T][H] fp32): partial sums of a shared-expert
// output, added (in order) with weight 1 before the routed rows.  inv ==
// nullptr: y is in (token, slot) order (row t*k + j), else in expert order
// (row inv[t*k + j]).
hipError_t launch_combine(const uint16_t *y, const int32_t *inv, const float *w, const float *y_sh32, int nsplit,
                          uint16_t *out, int T, int H, int k, hipStream_t st);

#ifdef MOE_DEBUG
// Bounds-check records of the MOE_DEBUG build, one per source file: rec[0]
// violations, rec[1] source line of the first; each read clears the record.
hipError_t debug_read_route(uint32_t *rec);
hipError_t debug_read_permute(uint32_t *rec);
hipError_t debug_read_gemm(uint32_t *rec);
hipError_t debug_read_combine(uint32_t *rec);
hipError_t debug_read_quant(uint32_t *rec);
#endif

}  // namespace moe
