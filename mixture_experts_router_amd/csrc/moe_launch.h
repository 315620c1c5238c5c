// Internal launchers of the MoE kernels (host side, called by the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kChunk = 1024;   // assignments per permutation block

hipError_t launch_router_gemm(const uint16_t *x, const uint16_t *wr, const float *bias,
                              float *logits, int T, int H, int E, hipStream_t st);
hipError_t launch_topk(const float *logits, int32_t *ids, float *w, int T, int E, int k,
                       hipStream_t st);
hipError_t launch_permute(const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_ids, int32_t *inv, int32_t *block_hist, int A, int E,
                          hipStream_t st);
hipError_t launch_gather_rows(const uint16_t *x, const int32_t *sorted_ids, uint16_t *x_perm,
                              int A, int H, int k, hipStream_t st);
hipError_t launch_gateup(const uint16_t *x, const int32_t *sorted_ids, int k, const int32_t *offsets,
                         const void *w, const uint8_t *scales, uint16_t *h, int A, int H, int E, int I,
                         bool mx, hipStream_t st);
hipError_t launch_down(const uint16_t *h, const int32_t *offsets, const void *w, const uint8_t *scales,
                       uint16_t *y, int A, int H, int E, int I, bool mx, hipStream_t st);
hipError_t launch_combine(const uint16_t *y, const int32_t *inv, const float *w, uint16_t *out, int T,
                          int H, int k, hipStream_t st);

}  // namespace moe
