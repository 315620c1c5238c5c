// C ABI of the MoE layer: argument checks (host only, before any HIP call),
// workspace layout and the kernel sequence of moe_forward.
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe.h"
#include "../../include/moe_debug.h"
#include "moe_launch.h"

// Scratch of moe_forward_noalloc: the library's own device memory, one copy
// on every GPU the library runs on, held until the process ends.  In host
// code this name is only a stand-in for the symbol; the device address of
// each GPU's copy comes from hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool is_nvfp4(const moe_shape *s) { return s->w_format == MOE_W_NVFP4 || s->w_format == MOE_W_NVFP4_A4; }

int check_shape(const moe_shape *s) {
    if (!s) return MOE_ERR_INVALID_ARGUMENT;
    if (s->T < 1 || s->H < 1 || s->E < 1 || s->k < 1 || s->I < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (s->k > s->E) return MOE_ERR_INVALID_ARGUMENT;
    if (s->w_format != MOE_W_BF16 && s->w_format != MOE_W_MXFP4 && s->w_format != MOE_W_MXFP4_A4 &&
        s->w_format != MOE_W_NVFP4 && s->w_format != MOE_W_NVFP4_A4)
        return MOE_ERR_UNSUPPORTED;
    if (s->H % 64 != 0 || s->I % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (s->E > 1024 || s->k > 32) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)s->T * s->k >= (int64_t{1} << 30)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int num_blocks(const moe_shape *s) {
    const int64_t A = (int64_t)s->T * s->k;
    return (int)((A + moe::kChunk - 1) / moe::kChunk);
}

size_t permute_ws(const moe_shape *s) { return round_up((size_t)num_blocks(s) * s->E * sizeof(int32_t)); }

// fp32 chunk partials of the split-K router (few tokens only).
size_t route_ws(const moe_shape *s) {
    if (!moe::router_uses_partials(s->T)) return 0;
    return round_up((size_t)moe::router_chunks(s->H) * s->T * s->E * sizeof(float));
}

int launch_route(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *bias,
                 float *logits, int32_t *ids, float *w, float *part, hipStream_t hs) {
    if (moe::router_uses_partials(s->T)) {
        if (moe::launch_router_partials(x, w_router, part, s->T, s->H, s->E, hs) != hipSuccess) return MOE_ERR_HIP;
        return moe::launch_topk(part, moe::router_chunks(s->H), bias, logits, ids, w, s->T, s->E, s->k, hs) ==
                       hipSuccess ? MOE_OK : MOE_ERR_HIP;
    }
    if (moe::launch_router_dense(x, w_router, bias, logits, s->T, s->H, s->E, hs) != hipSuccess) return MOE_ERR_HIP;
    return moe::launch_topk(nullptr, 0, nullptr, logits, ids, w, s->T, s->E, s->k, hs) == hipSuccess ? MOE_OK
                                                                                                      : MOE_ERR_HIP;
}

// Weight pointers: bf16 weights must be 16-byte aligned and come without
// scales; MXFP4 codes must be 4-byte aligned and come with scales.
int check_weights(const moe_shape *s, const void *w, const uint8_t *scales) {
    if (!w) return MOE_ERR_INVALID_ARGUMENT;
    if (s->w_format == MOE_W_BF16) {
        if (scales || !al16(w)) return MOE_ERR_INVALID_ARGUMENT;
    } else {
        // W4A4 streams the codes with 16-byte loads and the scales in pairs
        if (!scales || !(s->w_format == MOE_W_MXFP4_A4 ? al16(w) : al4(w))) return MOE_ERR_INVALID_ARGUMENT;
        if (s->w_format == MOE_W_MXFP4_A4 && (reinterpret_cast<uintptr_t>(scales) & 1u))
            return MOE_ERR_INVALID_ARGUMENT;
        // NVFP4: the fp32 header and one 32-bit load of 4 scales per row and step
        if (is_nvfp4(s) && !al4(scales)) return MOE_ERR_INVALID_ARGUMENT;
    }
    return MOE_OK;
}

// The grouped GEMMs' view of an expert weight argument: format, block
// scales, (NVFP4) the per-expert fp32 scales in front of them and (NVFP4
// activations) the activations' fp32 input scale that follows those.
struct WeightView {
    moe::WeightFormat fmt;
    const uint8_t *scales;
    const float *global;
    const float *input;
};

WeightView weight_view(const moe_shape *s, const uint8_t *scales) {
    if (is_nvfp4(s)) {
        const float *head = reinterpret_cast<const float *>(scales);
        return {moe::WeightFormat::kNVFP4, scales + MOE_NVFP4_HEADER_BYTES(s->E), head,
                s->w_format == MOE_W_NVFP4_A4 ? head + s->E : nullptr};
    }
    if (s->w_format == MOE_W_MXFP4) return {moe::WeightFormat::kMXFP4, scales, nullptr, nullptr};
    return {moe::WeightFormat::kBF16, scales, nullptr, nullptr};
}

struct Workspace {
    uint32_t *done;   // completion counter of the single-launch few-token routing
    float *part;
    float *logits;
    int32_t *ids;
    float *w;
    int32_t *counts, *offsets, *block_hist, *sorted_ids, *inv;
    uint16_t *h, *y;
    uint8_t *xq, *xs, *hq, *hs;   // W4A4 only: MXFP4 codes and scales of x and h
    uint16_t *xf;                 // NVFP4 activations only: x decoded after quantisation [T][H]
    uint16_t *h_sh;          // dense MLP (I_sh > 0 only): h rows [T][I_sh]
    float *y_sh32;           // and its down partial sums [nsplit][T][H]
    size_t bytes;
};

Workspace carve(const moe_shape *s, void *base, int I_sh = 0) {
    const size_t T = s->T, E = s->E, A = T * s->k;
    char *p = static_cast<char *>(base);
    size_t off = 0;
    Workspace w{};
    auto take = [&](size_t bytes) {
        char *q = p ? p + off : nullptr;
        off += round_up(bytes);
        return q;
    };
    w.done = reinterpret_cast<uint32_t *>(take(MOE_WS_ZERO_BYTES));
    w.part = reinterpret_cast<float *>(take(route_ws(s)));
    w.logits = reinterpret_cast<float *>(take(T * E * sizeof(float)));
    w.ids = reinterpret_cast<int32_t *>(take(A * sizeof(int32_t)));
    w.w = reinterpret_cast<float *>(take(A * sizeof(float)));
    w.counts = reinterpret_cast<int32_t *>(take(E * sizeof(int32_t)));
    w.offsets = reinterpret_cast<int32_t *>(take((E + 1) * sizeof(int32_t)));
    w.block_hist = reinterpret_cast<int32_t *>(take((size_t)num_blocks(s) * E * sizeof(int32_t)));
    w.sorted_ids = reinterpret_cast<int32_t *>(take(A * sizeof(int32_t)));
    w.inv = reinterpret_cast<int32_t *>(take(A * sizeof(int32_t)));
    w.h = reinterpret_cast<uint16_t *>(take(A * s->I * sizeof(uint16_t)));
    w.y = reinterpret_cast<uint16_t *>(take(A * s->H * sizeof(uint16_t)));
    const bool a4 = s->w_format == MOE_W_MXFP4_A4;
    w.xq = a4 ? reinterpret_cast<uint8_t *>(take(T * (size_t)s->H / 2)) : nullptr;
    w.xs = a4 ? reinterpret_cast<uint8_t *>(take(T * (size_t)s->H / 32)) : nullptr;
    w.hq = a4 ? reinterpret_cast<uint8_t *>(take(A * (size_t)s->I / 2)) : nullptr;
    w.hs = a4 ? reinterpret_cast<uint8_t *>(take(A * (size_t)s->I / 32)) : nullptr;
    w.xf = s->w_format == MOE_W_NVFP4_A4 ? reinterpret_cast<uint16_t *>(take(T * (size_t)s->H * 2)) : nullptr;
    w.h_sh = I_sh > 0 ? reinterpret_cast<uint16_t *>(take(T * (size_t)I_sh * sizeof(uint16_t))) : nullptr;
    w.y_sh32 = I_sh > 0 ? reinterpret_cast<float *>(take((size_t)moe::shared_splits(I_sh, s->I) * T * s->H *
                                                          sizeof(float)))
                        : nullptr;
    w.bytes = off;
    return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Device address of `scratch` on each device, looked up once per device
// with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

__global__ void zero_words_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The current device's scratch.  The first call on a device also clears its
// completion counters (the first MOE_WS_ZERO_BYTES) with a fill kernel on
// `hs`, ahead of the caller's kernels on that stream; every later call
// leaves them zero.
int noalloc_scratch(hipStream_t hs, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        constexpr int words = MOE_WS_ZERO_BYTES / 4;
        zero_words_kernel<<<1, words, 0, hs>>>(static_cast<uint32_t *>(p), words);
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

// Every argument check of moe_forward / moe_forward_shared except the
// workspace's (host only, launches nothing).
static int forward_checks(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *router_bias,
                          const void *w_gate_up, const uint8_t *gu_scales, const void *w_down,
                          const uint8_t *d_scales, int32_t I_sh, const void *w_sh_gate_up,
                          const uint8_t *sh_gu_scales, const void *w_sh_down, const uint8_t *sh_d_scales,
                          const uint16_t *out, const int32_t *topk_ids_out, const float *topk_w_out,
                          const moe_event_t *stage_events) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (I_sh < 0) return MOE_ERR_INVALID_ARGUMENT;
    const bool a4 = s->w_format == MOE_W_MXFP4_A4;
    if (I_sh > 0) {
        if (a4 || is_nvfp4(s) || I_sh % 64 != 0) return MOE_ERR_UNSUPPORTED;
        if ((st = check_weights(s, w_sh_gate_up, sh_gu_scales)) != MOE_OK) return st;
        if ((st = check_weights(s, w_sh_down, sh_d_scales)) != MOE_OK) return st;
    }
    if (!x || !w_router || !out) return MOE_ERR_INVALID_ARGUMENT;
    if (!al16(x) || !al16(w_router) || !al16(out)) return MOE_ERR_INVALID_ARGUMENT;
    if (router_bias && !al4(router_bias)) return MOE_ERR_INVALID_ARGUMENT;
    if ((topk_ids_out && !al4(topk_ids_out)) || (topk_w_out && !al4(topk_w_out)))
        return MOE_ERR_INVALID_ARGUMENT;
    if ((st = check_weights(s, w_gate_up, gu_scales)) != MOE_OK) return st;
    if ((st = check_weights(s, w_down, d_scales)) != MOE_OK) return st;
    if (stage_events)
        for (int i = 0; i <= MOE_FORWARD_STAGES; ++i)
            if (!stage_events[i]) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

// The kernel sequence of the layer on checked arguments and a workspace of
// at least carve(s, nullptr, I_sh).bytes.
static int forward_launch(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *router_bias,
                          const void *w_gate_up, const uint8_t *gu_scales, const void *w_down,
                          const uint8_t *d_scales, int32_t I_sh, const void *w_sh_gate_up,
                          const uint8_t *sh_gu_scales, const void *w_sh_down, const uint8_t *sh_d_scales,
                          uint16_t *out, int32_t *topk_ids_out, float *topk_w_out, void *ws, moe_stream_t stream,
                          const moe_event_t *stage_events) {
    int st = MOE_OK;
    const bool a4 = s->w_format == MOE_W_MXFP4_A4;
    Workspace w = carve(s, ws, I_sh);
    int32_t *ids = topk_ids_out ? topk_ids_out : w.ids;
    float *wts = topk_w_out ? topk_w_out : w.w;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int T = s->T, H = s->H, E = s->E, k = s->k, I = s->I, A = T * k;
    const WeightView gu = weight_view(s, gu_scales), dn = weight_view(s, d_scales);

    int stage = 0;
    auto mark = [&]() -> int {
        if (!stage_events) return MOE_OK;
        return hip_status(hipEventRecord(static_cast<hipEvent_t>(stage_events[stage++]), hs));
    };
    if ((st = mark()) != MOE_OK) return st;
    if (moe::route_permute_fits(T, k)) {
        // few tokens: router, top-k and the permutation in one launch (the
        // permute stage is empty)
        st = hip_status(moe::launch_route_permute(x, w_router, w.part, w.done, router_bias, w.logits, ids, wts,
                                                  w.counts, w.offsets, w.sorted_ids, w.inv, T, H, E, k, hs));
        if (st != MOE_OK || (st = mark()) != MOE_OK) return st;
        if ((st = mark()) != MOE_OK) return st;
    } else {
        st = launch_route(s, x, w_router, router_bias, w.logits, ids, wts, w.part, hs);
        if (st != MOE_OK || (st = mark()) != MOE_OK) return st;
        st = hip_status(
            moe::launch_permute(ids, w.counts, w.offsets, w.sorted_ids, w.inv, w.block_hist, A, E, hs));
        if (st != MOE_OK || (st = mark()) != MOE_OK) return st;
    }
    if (a4) {
        // W4A4: x and h quantised to MXFP4 before their matmuls (the
        // quantisations belong to the gate/up and down stages)
        st = hip_status(moe::launch_quantize_mx(x, T, H, w.xq, w.xs, hs));
        if (st == MOE_OK)
            st = hip_status(moe::launch_gateup_a4(w.xq, w.xs, w.sorted_ids, k, w.offsets, w_gate_up, gu_scales, w.h,
                                                  A, H, E, I, hs));
        if (st != MOE_OK || (st = mark()) != MOE_OK) return st;
        st = hip_status(moe::launch_quantize_mx(w.h, A, I, w.hq, w.hs, hs));
        if (st == MOE_OK)
            st = hip_status(
                moe::launch_down_a4(w.hq, w.hs, w.offsets, w_down, d_scales, w.y, w.sorted_ids, A, H, E, I, hs));
        if (st != MOE_OK || (st = mark()) != MOE_OK) return st;
        st = hip_status(moe::launch_combine(w.y, nullptr, wts, nullptr, 0, out, T, H, k, hs));
        if (st != MOE_OK) return st;
        return mark();
    }
    // NVFP4 activations: x and h quantised to NVFP4 (relative to the input
    // scales in the weights' scale headers) and decoded without those scales,
    // which the GEMM epilogues apply with the weights' (both quantisations
    // belong to the stages that multiply them; h is quantised in place)
    const bool nv_a4 = s->w_format == MOE_W_NVFP4_A4;
    const uint16_t *x_mm = x;
    if (nv_a4) {
        st = hip_status(moe::launch_quantize_nv(x, T, H, gu.input, nullptr, nullptr, w.xf, hs));
        if (st != MOE_OK) return st;
        x_mm = w.xf;
    }
    // the shared expert (if any) is an extra group of the same two launches
    const moe::SharedGroup sh_gu{x, w_sh_gate_up, sh_gu_scales, w.h_sh, nullptr, T, I_sh};
    const moe::SharedGroup sh_d{w.h_sh, w_sh_down, sh_d_scales, nullptr, w.y_sh32, T, I_sh};
    st = hip_status(moe::launch_gateup(x_mm, w.sorted_ids, k, w.offsets, w_gate_up, gu.scales, gu.global, gu.input,
                                       w.h, A, H, E, I, gu.fmt, I_sh > 0 ? &sh_gu : nullptr, hs));
    if (st != MOE_OK || (st = mark()) != MOE_OK) return st;
    if (nv_a4 && (st = hip_status(moe::launch_quantize_nv(w.h, A, I, dn.input, nullptr, nullptr, w.h, hs))) != MOE_OK)
        return st;
    // y in (token, slot) order: the combine reads each token's k rows
    // without a lookup of their positions first
    st = hip_status(moe::launch_down(w.h, w.offsets, w_down, dn.scales, dn.global, dn.input, w.y, w.sorted_ids, A, H,
                                     E, I, dn.fmt, I_sh > 0 ? &sh_d : nullptr, hs));
    if (st != MOE_OK || (st = mark()) != MOE_OK) return st;
    st = hip_status(moe::launch_combine(w.y, nullptr, wts, w.y_sh32, I_sh > 0 ? moe::shared_splits(I_sh, I) : 0, out,
                                        T, H, k, hs));
    if (st != MOE_OK) return st;
    return mark();
}

static int forward_impl(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *router_bias,
                        const void *w_gate_up, const uint8_t *gu_scales, const void *w_down, const uint8_t *d_scales,
                        int32_t I_sh, const void *w_sh_gate_up, const uint8_t *sh_gu_scales, const void *w_sh_down,
                        const uint8_t *sh_d_scales, uint16_t *out, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                        size_t ws_bytes, moe_stream_t stream, const moe_event_t *stage_events) {
    int st = forward_checks(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, I_sh, w_sh_gate_up,
                            sh_gu_scales, w_sh_down, sh_d_scales, out, topk_ids_out, topk_w_out, stage_events);
    if (st != MOE_OK) return st;
    const size_t need = carve(s, nullptr, I_sh).bytes;
    if (!ws || ws_bytes < need || !al16(ws)) return MOE_ERR_WORKSPACE;
    return forward_launch(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, I_sh, w_sh_gate_up,
                          sh_gu_scales, w_sh_down, sh_d_scales, out, topk_ids_out, topk_w_out, ws, stream,
                          stage_events);
}

extern "C" {

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported size or format";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP launch or event call failed";
        case MOE_ERR_SCRATCH_TOO_SMALL:
            return "shape needs more scratch than moe_forward_noalloc holds (MOE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

size_t moe_workspace_bytes(const moe_shape *s) {
    if (check_shape(s) != MOE_OK) return 0;
    return carve(s, nullptr).bytes;
}

size_t moe_route_workspace_bytes(const moe_shape *s) {
    if (check_shape(s) != MOE_OK) return 0;
    return route_ws(s);
}

size_t moe_permute_workspace_bytes(const moe_shape *s) {
    if (check_shape(s) != MOE_OK) return 0;
    return permute_ws(s);
}

int moe_route(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *router_bias,
              float *logits, int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, moe_stream_t stream) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
    if (!al4(logits) || !al4(topk_ids) || !al4(topk_w)) return MOE_ERR_INVALID_ARGUMENT;
    if (x) {
        if (!w_router || !al16(x) || !al16(w_router)) return MOE_ERR_INVALID_ARGUMENT;
        if (router_bias && !al4(router_bias)) return MOE_ERR_INVALID_ARGUMENT;
        const size_t need = route_ws(s);
        if (need && (!ws || ws_bytes < need || !al4(ws))) return MOE_ERR_WORKSPACE;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (x) return launch_route(s, x, w_router, router_bias, logits, topk_ids, topk_w, static_cast<float *>(ws), hs);
    return moe::launch_topk(nullptr, 0, nullptr, logits, topk_ids, topk_w, s->T, s->E, s->k, hs) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

int moe_permute(const moe_shape *s, const int32_t *topk_ids, const uint16_t *x, int32_t *counts,
                int32_t *offsets, int32_t *sorted_ids, int32_t *inv, uint16_t *x_perm, void *ws,
                size_t ws_bytes, moe_stream_t stream) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (!topk_ids || !counts || !offsets || !sorted_ids || !inv) return MOE_ERR_INVALID_ARGUMENT;
    if (!al4(topk_ids) || !al4(counts) || !al4(offsets) || !al4(sorted_ids) || !al4(inv))
        return MOE_ERR_INVALID_ARGUMENT;
    if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    if (x && (!al16(x) || !al16(x_perm))) return MOE_ERR_INVALID_ARGUMENT;
    if (!ws || ws_bytes < permute_ws(s) || !al4(ws)) return MOE_ERR_WORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int A = s->T * s->k;
    st = hip_status(moe::launch_permute(topk_ids, counts, offsets, sorted_ids, inv,
                                        static_cast<int32_t *>(ws), A, s->E, hs));
    if (st != MOE_OK || !x) return st;
    return hip_status(moe::launch_gather_rows(x, sorted_ids, x_perm, A, s->H, s->k, hs));
}

int moe_grouped_gemm_gateup(const moe_shape *s, const uint16_t *x, const int32_t *sorted_ids,
                            const int32_t *offsets, const void *w_gate_up, const uint8_t *gu_scales,
                            uint16_t *h, moe_stream_t stream) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (!x || !offsets || !h) return MOE_ERR_INVALID_ARGUMENT;
    if (!al16(x) || !al16(h) || !al4(offsets)) return MOE_ERR_INVALID_ARGUMENT;
    if (sorted_ids && !al4(sorted_ids)) return MOE_ERR_INVALID_ARGUMENT;
    if ((st = check_weights(s, w_gate_up, gu_scales)) != MOE_OK) return st;
    if (s->w_format == MOE_W_MXFP4_A4 || s->w_format == MOE_W_NVFP4_A4) return MOE_ERR_UNSUPPORTED;
    const WeightView wv = weight_view(s, gu_scales);
    return hip_status(moe::launch_gateup(x, sorted_ids, s->k, offsets, w_gate_up, wv.scales, wv.global, nullptr, h,
                                         s->T * s->k, s->H, s->E, s->I, wv.fmt, nullptr,
                                         static_cast<hipStream_t>(stream)));
}

int moe_grouped_gemm_down(const moe_shape *s, const uint16_t *h, const int32_t *offsets, const void *w_down,
                          const uint8_t *d_scales, uint16_t *y, moe_stream_t stream) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (!h || !offsets || !y) return MOE_ERR_INVALID_ARGUMENT;
    if (!al16(h) || !al16(y) || !al4(offsets)) return MOE_ERR_INVALID_ARGUMENT;
    if ((st = check_weights(s, w_down, d_scales)) != MOE_OK) return st;
    if (s->w_format == MOE_W_MXFP4_A4 || s->w_format == MOE_W_NVFP4_A4) return MOE_ERR_UNSUPPORTED;
    const WeightView wv = weight_view(s, d_scales);
    return hip_status(moe::launch_down(h, offsets, w_down, wv.scales, wv.global, nullptr, y, nullptr, s->T * s->k,
                                       s->H, s->E, s->I, wv.fmt, nullptr, static_cast<hipStream_t>(stream)));
}

int moe_combine(const moe_shape *s, const uint16_t *y, const int32_t *inv, const float *topk_w,
                uint16_t *out, moe_stream_t stream) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (!y || !inv || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
    if (!al16(y) || !al16(out) || !al4(inv) || !al4(topk_w)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_combine(y, inv, topk_w, nullptr, 0, out, s->T, s->H, s->k,
                                          static_cast<hipStream_t>(stream)));
}

int moe_forward(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *router_bias,
                const void *w_gate_up, const uint8_t *gu_scales, const void *w_down, const uint8_t *d_scales,
                uint16_t *out, int32_t *topk_ids_out, float *topk_w_out, void *ws, size_t ws_bytes,
                moe_stream_t stream, const moe_event_t *stage_events) {
    return forward_impl(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, 0, nullptr, nullptr,
                        nullptr, nullptr, out, topk_ids_out, topk_w_out, ws, ws_bytes, stream, stage_events);
}

int moe_forward_shared(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *router_bias,
                       const void *w_gate_up, const uint8_t *gu_scales, const void *w_down, const uint8_t *d_scales,
                       int32_t I_sh, const void *w_sh_gate_up, const uint8_t *sh_gu_scales, const void *w_sh_down,
                       const uint8_t *sh_d_scales, uint16_t *out, int32_t *topk_ids_out, float *topk_w_out,
                       void *ws, size_t ws_bytes, moe_stream_t stream, const moe_event_t *stage_events) {
    if (I_sh <= 0) return MOE_ERR_INVALID_ARGUMENT;
    return forward_impl(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, I_sh, w_sh_gate_up,
                        sh_gu_scales, w_sh_down, sh_d_scales, out, topk_ids_out, topk_w_out, ws, ws_bytes, stream,
                        stage_events);
}

int moe_quantize_mx(const uint16_t *src, int64_t rows, int32_t K, uint8_t *codes, uint8_t *scales,
                    moe_stream_t stream) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return rows < 0 || K <= 0 ? MOE_ERR_INVALID_ARGUMENT : MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!src || !codes || !scales || !al16(src) || !al16(codes)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_quantize_mx(src, rows, K, codes, scales, static_cast<hipStream_t>(stream)));
}

int moe_forward_noalloc(const moe_shape *s, const uint16_t *x, const uint16_t *w_router, const float *router_bias,
                        const void *w_gate_up, const uint8_t *gu_scales, const void *w_down, const uint8_t *d_scales,
                        uint16_t *out, int32_t *topk_ids_out, float *topk_w_out, moe_stream_t stream) {
    int st = forward_checks(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, 0, nullptr,
                            nullptr, nullptr, nullptr, out, topk_ids_out, topk_w_out, nullptr);
    if (st != MOE_OK) return st;
    if (carve(s, nullptr).bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_TOO_SMALL;
    void *ws = nullptr;
    if ((st = noalloc_scratch(static_cast<hipStream_t>(stream), &ws)) != MOE_OK) return st;
    return forward_launch(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, 0, nullptr, nullptr,
                          nullptr, nullptr, out, topk_ids_out, topk_w_out, ws, stream, nullptr);
}

int moe_quantize_nv(const uint16_t *src, int64_t rows, int32_t K, const float *input_scale, uint8_t *codes,
                    uint8_t *scales, moe_stream_t stream) {
    if (rows < 0 || K <= 0) return MOE_ERR_INVALID_ARGUMENT;
    if (K % 16 != 0) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!src || !input_scale || !codes || !scales || !al16(src) || !al4(input_scale) ||
        (reinterpret_cast<uintptr_t>(codes) & 7u))
        return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_quantize_nv(src, rows, K, input_scale, codes, scales, nullptr,
                                              static_cast<hipStream_t>(stream)));
}

#ifdef MOE_DEBUG
int moe_debug_bounds(uint32_t *violations, uint32_t *where) {
    if (!violations || !where) return MOE_ERR_INVALID_ARGUMENT;
    hipError_t (*const readers[])(uint32_t *) = {moe::debug_read_route, moe::debug_read_permute,
                                                 moe::debug_read_gemm, moe::debug_read_combine,
                                                 moe::debug_read_quant};
    *violations = 0;
    *where = 0;
    for (int i = 0; i < 5; ++i) {
        uint32_t rec[2] = {0u, 0u};
        if (readers[i](rec) != hipSuccess) return MOE_ERR_HIP;
        if (rec[0] && !*violations) *where = 100000u * (uint32_t)(i + 1) + rec[1];
        *violations += rec[0];
    }
    return MOE_OK;
}
#endif

size_t moe_workspace_shared_bytes(const moe_shape *s, int32_t I_sh) {
    if (check_shape(s) != MOE_OK || I_sh <= 0 || I_sh % 64 != 0) return 0;
    return carve(s, nullptr, I_sh).bytes;
}

}  // extern "C"
