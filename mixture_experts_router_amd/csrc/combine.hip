// Weighted combine: out[t] = sum_{j<k} w[t, j] * y[inv[t*k + j]] (y in expert
// order), or y[t*k + j] (y in (token, slot) order, as the whole layer stores
// it), summed in fp32 in ascending j and rounded to bf16 once.  This is the local-expert sum
// that the decode path of the pages all-reduces across expert-parallel
// ranks (Gemma-4-26B-A4B optimisation report, section 6.1, MoE row).  Each
// output element is owned by one lane, so there are no atomics and the
// result is bitwise reproducible.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

// One wave per (token, 512 consecutive outputs); each lane owns 8
// consecutive outputs (16 bytes).  The token's k rows and weights are
// wave-uniform (scalar loads); the row loads go out in batches of 8.  A
// token's pieces are consecutive blocks, so the pieces of each gathered row
// are requested together rather than one row-piece per token across the
// whole grid.
__global__ __launch_bounds__(64) void combine_kernel(const uint16_t *__restrict__ y,
                                                     const int32_t *__restrict__ inv,
                                                     const float *__restrict__ w,
                                                     const float *__restrict__ y_sh32, int nsplit,
                                                     uint16_t *__restrict__ out, int T, int H, int k, int npieces) {
    const int t = blockIdx.x / npieces, piece = blockIdx.x - t * npieces;
    const int c = piece * 64 + threadIdx.x;   // 16-byte chunk of the row
    if (c >= H / 8) return;
    combine_chunk(y, inv, w, y_sh32, nsplit, out, t, c * 8, T, H, k);
}

hipError_t launch_combine(const uint16_t *y, const int32_t *inv, const float *w, const float *y_sh32, int nsplit,
                          uint16_t *out, int T, int H, int k, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int npieces = (H / 8 + 63) / 64;
    const long long blocks = (long long)T * npieces;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    combine_kernel<<<dim3((unsigned)blocks), 64, 0, st>>>(y, inv, w, y_sh32, nsplit, out, T, H, k, npieces);
    return hipGetLastError();
}

#ifdef MOE_DEBUG
MOE_DEBUG_READER(debug_read_combine)
#endif

}  // namespace moe
