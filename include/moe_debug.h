/*
 * moe_debug.h -- the bounds-checked build of the MoE layer library
 * (libmoe_debug.so, compiled with MOE_DEBUG).
 *
 * In that build every kernel checks each global address it forms from
 * indices (token rows gathered through sorted_ids, expert weight and scale
 * rows, tile outputs, scatter positions, combine rows, chunk sums) against
 * the extent of the buffer it must lie in.  An access outside is not made:
 * it is redirected to the buffer's first byte and recorded, so a wrong
 * index shows up as a counted violation instead of a memory fault or a
 * silent overwrite.  The entry points of include/moe.h behave as in the
 * release library otherwise (slower); the release library does not export
 * this function.
 */
#ifndef MOE_DEBUG_H
#define MOE_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_debug_bounds -- read and clear the bounds-check records of all kernels
 * on the current device.  Synchronises the device (a blocking copy).
 *   violations  out: accesses redirected since the last read
 *   where       out: 0 if none, else 100000 * f + line: the source file f
 *               (1 routing, 2 permutation, 3 grouped GEMM, 4 combine,
 *               5 quantisers) and line of the first violation in it
 * Returns MOE_OK, MOE_ERR_INVALID_ARGUMENT (NULL pointer) or MOE_ERR_HIP.
 */
int moe_debug_bounds(uint32_t *violations, uint32_t *where);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DEBUG_H */
