/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts FFN layer.
 *
 * The layer (Gemma-4-26B-A4B optimisation report, section 1 model overview:
 * each decoder block has an MoE of 128 experts with top-8 routing, expert
 * intermediate 704 and a GEGLU activation; Gemma-4-26B-A4B-NVFP4 Ascend
 * verification report, section 2.1: hidden 2816, gelu_pytorch_tanh, bf16):
 *
 *   route    logits = x W_r^T (+ b); per token the top-k experts and their
 *            renormalised softmax weights         (report, section 5, router op)
 *   permute  per-expert counts, offsets and the expert-grouped order of the
 *            (token, slot) assignments; optional gathered copy of x
 *                                                 (report, section 6.1, dispatch)
 *   gate/up  per expert, h = gelu_tanh(X W_gate^T) * (X W_up^T)    (GEGLU)
 *   down     per expert, y = h W_down^T
 *   combine  out[t] = sum_j w[t, j] y[inv[t*k + j]]  (report, section 6.1,
 *            the local-expert weighted sum)
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers on the current HIP device,
 *     row-major, densely packed.  bf16 values travel as uint16_t bit patterns.
 *   - Weights are K-contiguous: w_router [E][H]; w_gate_up [E][2I][H] whose
 *     rows 0..I-1 are the gate and rows I..2I-1 the up projection; w_down
 *     [E][H][I].  MXFP4 weights (w_format MOE_W_MXFP4) replace a bf16 row of
 *     K values by K/2 bytes of E2M1 codes (two per byte, the even K index in
 *     the low nibble) plus K/32 E8M0 scale bytes (value 2^(byte-127)); the
 *     E2M1/E8M0 encodings are the OCP Microscaling Formats v1.0 ones.  The
 *     router weight is always bf16.  Decoded weights must be normal bf16
 *     numbers (scale bytes 2..250 guarantee it); 0xFF scales are undefined.
 *     NVFP4 weights (w_format MOE_W_NVFP4, the format of the
 *     Gemma-4-26B-A4B-NVFP4 checkpoint of the verification report) have the
 *     same E2M1 codes with one FP8 E4M3 scale per 16 consecutive K values
 *     and one fp32 scale per expert matrix; a weight is E2M1(code) x
 *     E4M3(block scale) x matrix scale.  Their scale argument is one buffer:
 *     MOE_NVFP4_HEADER_BYTES(E) bytes holding the E fp32 matrix scales and
 *     the activation input scale (NVFP4_A4), then the E4M3 codes
 *     [E][rows][K/16].  E4M3 is the OCP 8-bit floating point
 *     format (exponent bias 7, largest value 448, no infinities); its NaN
 *     codes (0x7F, 0xFF) are undefined as scales.
 *   - Assignment a = t*k + j is slot j of token t.  A = T*k.
 *   - Routing: the k largest logits, ties to the lower expert index, slots in
 *     (logit descending, index ascending) order; w = softmax over the k
 *     selected logits.  Non-finite logits give undefined routing.
 *   - Expert-grouped order: position p of sorted_ids holds the assignment a;
 *     assignments of expert e occupy [offsets[e], offsets[e+1]) in ascending
 *     token order.  inv[a] = p.  Every token has exactly k assignments; no
 *     capacity limit, nothing dropped.  Empty experts read no weight bytes.
 *   - Arithmetic: bf16 inputs, fp32 accumulation; h, y and out are rounded
 *     to bf16 (nearest-even); the combine sums in fp32 in ascending j.  The
 *     router accumulates in fp32 over blocks of 256 products and adds the
 *     block sums in fp64 before the single rounding of each logit to fp32.
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     workspace.  The library allocates nothing and keeps no pointer after a
 *     call returns.  Inputs are never written.  (moe_forward_noalloc takes
 *     its workspace from a scratch buffer of the library instead: below.)
 *   - Execution: every call only enqueues kernels on `stream` (a hipStream_t;
 *     NULL is the null stream).  None synchronises or copies data to the
 *     host.  The entry points other than moe_forward_noalloc hold no global
 *     mutable state; their calls on different streams with disjoint outputs
 *     and workspaces may overlap.
 *   - Errors: the return value is a status.  Shape, pointer, alignment and
 *     workspace checks run on the host before any HIP call; a failing check
 *     launches nothing.  MOE_ERR_HIP reports a launch failure; faults during
 *     execution surface at the caller's next synchronisation.  No C++
 *     exception crosses this interface.
 *   - Supported sizes: H % 64 == 0, I % 64 == 0, 1 <= k <= min(E, 32),
 *     E <= 1024, T*k < 2^30.  Pointers to bf16 arrays, x_perm, h and y must
 *     be 16-byte aligned (W4A4 weight codes too), the other arrays 4-byte
 *     aligned (MXFP4 scales: any address, 2-byte aligned for W4A4; NVFP4
 *     scale buffers 4-byte aligned).  W4A4 gate/up weight scales that are
 *     8-byte aligned, with H % 256 == 0, are read 8 bytes per row and step
 *     (faster; the results are the same bits).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_shape {
    int32_t T;        /* tokens */
    int32_t H;        /* hidden size */
    int32_t E;        /* experts */
    int32_t k;        /* experts per token */
    int32_t I;        /* expert intermediate size */
    int32_t w_format; /* MOE_W_BF16, MOE_W_MXFP4, MOE_W_MXFP4_A4, MOE_W_NVFP4 or MOE_W_NVFP4_A4 */
} moe_shape;

/* Expert weight format.  MOE_W_MXFP4_A4 (W4A4): MXFP4 weights, and the
 * expert matmuls' activations -- x, and each expert's bf16 h -- quantised to
 * MXFP4 per 32 consecutive K values before they are multiplied (OCP MX v1.0
 * conversion: scale 2^(floor(log2 amax) - 2), clamped exponent, 2^0 for an
 * all-zero block; values to the nearest E2M1 code, ties to the even code,
 * saturating at 6), on the gfx950 block-scaled FP4 matrix instructions.
 * The router still reads the bf16 x.  The vLLM-Ascend Gemma4 tutorial,
 * section 3.1, names w4a4 MXFP4 checkpoints.  W4A4 runs through moe_forward
 * (no dense MLP) and moe_quantize_mx only; the per-step GEMM entry points
 * return MOE_ERR_UNSUPPORTED for it.  MOE_W_NVFP4: NVFP4 expert weights
 * (above) with bf16 activations, through moe_forward and the per-step GEMM
 * entry points; not with a dense MLP.  MOE_W_NVFP4_A4: NVFP4 weights and
 * NVFP4 activations (the Gemma-4-26B-A4B-NVFP4 verification report, section
 * 2.3: weights and activations 4-bit float in groups of 16): x, and each
 * expert's bf16 h, are quantised per 16 consecutive K values relative to the
 * activation's fp32 input scale g (a calibration constant, slot E of the
 * gate/up and down scale headers): block scale = the E4M3 value nearest to
 * amax / (6 g) (ties to the even code, 448 from 448 up), each value v /
 * (block scale * g) to the nearest E2M1 code (ties to the even code,
 * saturating at 6), decided in fp32 (moe_quantize_nv).  gfx950 has no FP4
 * matrix instruction with E4M3 scales: both operands are multiplied on the
 * bf16 matrix cores as their exact decoded values (E2M1 x E4M3 has at most
 * six significant bits), with fp32 sums scaled by the weight's matrix scale
 * times g.  Through moe_forward only; not with a dense MLP. */
enum { MOE_W_BF16 = 0, MOE_W_MXFP4 = 1, MOE_W_MXFP4_A4 = 2, MOE_W_NVFP4 = 3, MOE_W_NVFP4_A4 = 4 };

/* Bytes in front of the E4M3 codes of an NVFP4 scale buffer: the E fp32
 * matrix scales and one fp32 activation input scale (slot E, read by
 * MOE_W_NVFP4_A4 only), padded to a multiple of 256. */
#define MOE_NVFP4_HEADER_BYTES(E) (((((size_t)(E) + 1u) * 4u + 255u) / 256u) * 256u)

enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = -1, /* NULL pointer, T/H/E/I < 1, k < 1, k > E, misalignment */
    MOE_ERR_UNSUPPORTED = -2,      /* a size outside the supported set above */
    MOE_ERR_WORKSPACE = -3,        /* workspace NULL or smaller than required */
    MOE_ERR_HIP = -4,              /* a HIP launch or event call failed */
    MOE_ERR_SCRATCH_TOO_SMALL = -5 /* moe_forward_noalloc: the shape needs more than its scratch */
};

typedef void *moe_stream_t; /* hipStream_t */
typedef void *moe_event_t;  /* hipEvent_t */

/* Number of stages moe_forward times when given stage events. */
#define MOE_FORWARD_STAGES 5
/* Leading workspace bytes of moe_forward that must start out zero. */
#define MOE_WS_ZERO_BYTES 256

/*
 * moe_route -- router GEMM, top-k and softmax weights (report, section 5:
 * the router op fused as gating top-k softmax).
 *   x            [T][H] bf16, or NULL: then `logits` is an INPUT [T][E] fp32
 *                and w_router / router_bias are ignored
 *   w_router     [E][H] bf16 (required when x != NULL)
 *   router_bias  [E] fp32 or NULL
 *   logits       [T][E] fp32: output when x != NULL, input when x == NULL
 *   topk_ids     [T][k] int32 out;  topk_w [T][k] fp32 out (rows sum to 1)
 *   ws           device scratch of at least moe_route_workspace_bytes(s)
 *                (may be NULL when that is 0 or when x == NULL)
 */
int moe_route(const moe_shape *s, const uint16_t *x, const uint16_t *w_router,
              const float *router_bias, float *logits, int32_t *topk_ids,
              float *topk_w, void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_permute -- expert histogram, prefix scan and stable scatter: the
 * data-dependent split sizes and order of the dispatch (report, section 6.1).
 *   topk_ids     [T][k] int32 in, each in [0, E)
 *   counts       [E] int32 out;  offsets [E+1] int32 out (offsets[E] = T*k)
 *   sorted_ids   [T*k] int32 out; inv [T*k] int32 out
 *   x, x_perm    both NULL, or x [T][H] bf16 in and x_perm [T*k][H] bf16 out
 *                with x_perm[p] = x[sorted_ids[p] / k] (bitwise copy)
 *   ws           device scratch of at least moe_permute_workspace_bytes(s)
 */
int moe_permute(const moe_shape *s, const int32_t *topk_ids, const uint16_t *x,
                int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                int32_t *inv, uint16_t *x_perm, void *ws, size_t ws_bytes,
                moe_stream_t stream);

/*
 * moe_grouped_gemm_gateup -- per expert e with rows [offsets[e],
 * offsets[e+1]): G = X_e W_gu[e]^T (fp32), h = gelu_tanh(G[:, :I]) * G[:, I:]
 * rounded to bf16 (GEGLU, report, section 1; gelu_pytorch_tanh, verification
 * report, section 2.1).  gelu_tanh(z) = 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))).
 *   x            sorted_ids == NULL: x_perm [T*k][H] bf16, row p = assignment p
 *                sorted_ids != NULL: x [T][H] bf16, row p = x[sorted_ids[p] / k]
 *   sorted_ids   [T*k] int32 or NULL (see x)
 *   offsets      [E+1] int32
 *   w_gate_up    bf16 [E][2I][H], or MXFP4 / NVFP4 codes [E][2I][H/2]
 *   gu_scales    NULL for bf16; MXFP4 scales [E][2I][H/32]; NVFP4 scale
 *                buffer (E fp32, then E4M3 codes [E][2I][H/16])
 *   h            [T*k][I] bf16 out
 */
int moe_grouped_gemm_gateup(const moe_shape *s, const uint16_t *x,
                            const int32_t *sorted_ids, const int32_t *offsets,
                            const void *w_gate_up, const uint8_t *gu_scales,
                            uint16_t *h, moe_stream_t stream);

/*
 * moe_grouped_gemm_down -- per expert: y rows = h rows W_d[e]^T, fp32
 * accumulation, bf16 out.
 *   h            [T*k][I] bf16;  offsets [E+1] int32
 *   w_down       bf16 [E][H][I], or MXFP4 / NVFP4 codes [E][H][I/2]
 *   d_scales     NULL for bf16; MXFP4 scales [E][H][I/32]; NVFP4 scale
 *                buffer (E fp32, then E4M3 codes [E][H][I/16])
 *   y            [T*k][H] bf16 out
 */
int moe_grouped_gemm_down(const moe_shape *s, const uint16_t *h,
                          const int32_t *offsets, const void *w_down,
                          const uint8_t *d_scales, uint16_t *y,
                          moe_stream_t stream);

/*
 * moe_combine -- out[t] = sum_{j<k} topk_w[t][j] * y[inv[t*k+j]], fp32 sum
 * in ascending j, one bf16 rounding; no atomics, so bitwise reproducible.
 *   y [T*k][H] bf16; inv [T*k] int32; topk_w [T][k] fp32; out [T][H] bf16
 */
int moe_combine(const moe_shape *s, const uint16_t *y, const int32_t *inv,
                const float *topk_w, uint16_t *out, moe_stream_t stream);

/*
 * moe_forward -- the whole layer: route, permute (without materialising
 * x_perm: the gate/up GEMM gathers x rows itself), gate/up + GEGLU, down
 * (its rows stored in (token, slot) order, so the combine needs no inv
 * lookup), combine, all on `stream`, with a launch grid that depends only on the
 * shape (never on routing counts), no host synchronisation and no
 * device-to-host copy.
 *   weights and scales as for the steps above
 *   out           [T][H] bf16 out
 *   topk_ids_out  [T][k] int32 out or NULL;  topk_w_out [T][k] fp32 out or NULL
 *   ws            device scratch of at least moe_workspace_bytes(s), 16-byte
 *                 aligned.  Its first MOE_WS_ZERO_BYTES bytes hold completion
 *                 counters: they must be zero before the first call with this
 *                 workspace (allocate it zero-filled), and every call leaves
 *                 them zero again.  Calls that overlap in time must not share
 *                 a workspace.
 *   stage_events  NULL, or MOE_FORWARD_STAGES + 1 hipEvent_t recorded on
 *                 `stream` before the first stage and after each stage
 *                 (route, permute, gate/up, down, combine)
 */
int moe_forward(const moe_shape *s, const uint16_t *x, const uint16_t *w_router,
                const float *router_bias, const void *w_gate_up,
                const uint8_t *gu_scales, const void *w_down,
                const uint8_t *d_scales, uint16_t *out, int32_t *topk_ids_out,
                float *topk_w_out, void *ws, size_t ws_bytes,
                moe_stream_t stream, const moe_event_t *stage_events);

/*
 * moe_forward_shared -- moe_forward plus an always-on dense GEGLU MLP of
 * intermediate size I_sh applied to every token and added with weight 1 (the
 * decoder block runs a dense MLP next to the MoE: Gemma-4-26B-A4B
 * optimisation report, section 1, dense MLP of intermediate 2112; section 5,
 * its gate/up width 4224):
 *   out[t] = MLP(x[t]) + sum_j topk_w[t][j] * expert_j(x[t]),
 *   MLP(x) = (gelu_tanh(x Wg^T) * (x Wu^T)) Wd^T
 * The MLP runs as one more group inside the same two grouped GEMM launches;
 * its h and output rows are rounded to bf16 like the experts', and the
 * combine starts its fp32 sum from the MLP row.
 *   I_sh          > 0, multiple of 64
 *   w_sh_gate_up  [2*I_sh][H] (gate rows first) in the experts' format:
 *                 bf16 (sh_gu_scales NULL) or MXFP4 codes [2*I_sh][H/2] with
 *                 scales [2*I_sh][H/32]
 *   w_sh_down     [H][I_sh] likewise (sh_d_scales [H][I_sh/32] for MXFP4)
 *   ws            at least moe_workspace_shared_bytes(s, I_sh) bytes, with
 *                 the same zero-prefix rule as moe_forward
 *   other arguments, errors and execution as for moe_forward
 */
int moe_forward_shared(const moe_shape *s, const uint16_t *x,
                       const uint16_t *w_router, const float *router_bias,
                       const void *w_gate_up, const uint8_t *gu_scales,
                       const void *w_down, const uint8_t *d_scales,
                       int32_t I_sh, const void *w_sh_gate_up,
                       const uint8_t *sh_gu_scales, const void *w_sh_down,
                       const uint8_t *sh_d_scales, uint16_t *out,
                       int32_t *topk_ids_out, float *topk_w_out, void *ws,
                       size_t ws_bytes, moe_stream_t stream,
                       const moe_event_t *stage_events);

/*
 * moe_quantize_mx -- MXFP4 codes and E8M0 scales of bf16 rows, per 32
 * consecutive values (the W4A4 activation conversion described with
 * MOE_W_MXFP4_A4).
 *   src     [rows][K] bf16, 16-byte aligned; K > 0, K % 32 == 0
 *   codes   [rows][K/2] out, two codes per byte (even index low), 16-byte aligned
 *   scales  [rows][K/32] out, E8M0 bytes
 *   rows >= 0 (0 launches nothing)
 */
int moe_quantize_mx(const uint16_t *src, int64_t rows, int32_t K, uint8_t *codes,
                    uint8_t *scales, moe_stream_t stream);

/*
 * moe_forward_noalloc -- moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels, with the workspace taken from a
 * scratch buffer inside the library instead of an argument.  It calls no
 * allocating routine.
 *   arguments, layout and errors as for moe_forward (no workspace, no stage
 *   events); MOE_ERR_SCRATCH_TOO_SMALL, before any launch, when
 *   moe_workspace_bytes(s) > MOE_NOALLOC_SCRATCH_BYTES (64 MiB: the
 *   Gemma-4 layer shape up to about 1 100 tokens)
 * Scratch: one static device buffer of MOE_NOALLOC_SCRATCH_BYTES per GPU,
 * held by every GPU the library runs on until the process ends.  Its
 * address on the current device is looked up on the first call on that
 * device, which also enqueues a fill kernel on `stream` that clears its
 * completion counters; every call leaves them zero again.  All calls on one
 * GPU share its buffer, and it keeps the last call's contents: calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * undefined results, so order them on one stream or synchronise between
 * them.  Make the first call on each device outside graph capture.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_shape *s, const uint16_t *x, const uint16_t *w_router,
                        const float *router_bias, const void *w_gate_up,
                        const uint8_t *gu_scales, const void *w_down,
                        const uint8_t *d_scales, uint16_t *out, int32_t *topk_ids_out,
                        float *topk_w_out, moe_stream_t stream);

/*
 * moe_quantize_nv -- NVFP4 codes and E4M3 block scales of bf16 rows, per 16
 * consecutive values, relative to an fp32 input scale (the activation
 * conversion described with MOE_W_NVFP4_A4).
 *   src          [rows][K] bf16, 16-byte aligned; K > 0, K % 16 == 0
 *   input_scale  one fp32 (device), 4-byte aligned
 *   codes        [rows][K/2] out, two E2M1 codes per byte (even index low),
 *                8-byte aligned
 *   scales       [rows][K/16] out, E4M3 codes
 *   rows >= 0 (0 launches nothing)
 */
int moe_quantize_nv(const uint16_t *src, int64_t rows, int32_t K, const float *input_scale,
                    uint8_t *codes, uint8_t *scales, moe_stream_t stream);

/* Workspace bytes moe_forward needs for this shape; 0 for an invalid or
 * unsupported shape.  Monotone in T. */
size_t moe_workspace_bytes(const moe_shape *s);

/* Workspace bytes moe_forward_shared needs; 0 for an invalid shape or an
 * I_sh that is not a positive multiple of 64. */
size_t moe_workspace_shared_bytes(const moe_shape *s, int32_t I_sh);

/* Workspace bytes moe_route needs for this shape (0: none needed, or an
 * invalid shape).  Few tokens use a split-K router with per-chunk partial
 * sums; many tokens need no scratch. */
size_t moe_route_workspace_bytes(const moe_shape *s);

/* Workspace bytes moe_permute needs for this shape; 0 if invalid. */
size_t moe_permute_workspace_bytes(const moe_shape *s);

/* Static description of a status code; never NULL. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
