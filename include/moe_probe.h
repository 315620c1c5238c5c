/*
 * moe_probe.h -- load-only streaming probes (libmoe_probe.so).
 *
 * A measurement aid, not part of the layer: kernels that read bytes from
 * HBM through the same direct-to-LDS loads as the grouped GEMMs and do no
 * arithmetic, for a plain stream and for the launch shapes of the decode
 * gate/up and down GEMMs.  Their durations are what the chip delivers at
 * those shapes, the yardstick for the GEMMs' achieved bandwidth.  One probe
 * reads LDS only (16 waves per CU, conflict-free 16-byte reads): the LDS
 * read rate.  The layer library never loads this one.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of probes (kinds 0 .. count-1). */
int moe_probe_count(void);

/* Name of probe `kind` (a static string), NULL for an unknown kind. */
const char *moe_probe_name(int kind);

/* Bytes one launch of probe `kind` reads (from HBM, or from LDS for the LDS
 * probe), 0 for an unknown kind. */
size_t moe_probe_bytes(int kind);

/* Bytes of `buf` that probe `kind` reads from (0 for the LDS probe and for an
 * unknown kind). */
size_t moe_probe_footprint(int kind);

/*
 * moe_probe_launch -- enqueue one launch of probe `kind` on `stream`
 * (a hipStream_t, or NULL for the null stream); does not synchronise.
 *   buf        device buffer, 256-byte aligned, read only (non-NULL also
 *              for the LDS probe, which does not read it)
 *   buf_bytes  its length: at least moe_probe_footprint(kind)
 *   sink       device buffer of at least 1024 ints; each workgroup writes one
 *              (keeps the loads from being dropped)
 * Returns 0, -1 for an unknown kind, a NULL or misaligned pointer or a short
 * buffer (nothing launched), -2 if the launch failed.
 */
int moe_probe_launch(int kind, const void *buf, size_t buf_bytes, int *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
