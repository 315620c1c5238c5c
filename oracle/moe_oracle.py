"""Plain, slow fp64 CPU oracle of the Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check of the package
entry module and the CPU-baseline leg of the benchmark may import this
module.  It shares no code with the HIP path and imports nothing from it.

What the layer computes (Gemma-4-26B-A4B optimisation report, section 1 model
overview: every decoder block has an MoE with 128 experts, top-8 routing,
expert intermediate 704 and a GEGLU activation; section 5 names the fused
router op that does top-k + softmax over the router logits; section 6.1
describes the dispatch of tokens grouped by expert and the weighted combine
of the expert outputs; Gemma-4-26B-A4B-NVFP4 Ascend verification report,
section 2.1 model architecture parameters: hidden 2816, activation
gelu_pytorch_tanh):

  O1  decode every bf16 input exactly to fp64
  O2  router logits L = x W_r^T (+ b)
  O3  per token, the k experts with the largest logits; ties go to the lower
      expert index; slots ordered by (logit descending, index ascending)
  O4  routing weights: softmax over the k selected logits (renormalised top-k)
  O5  per-expert counts and their exclusive prefix sum (offsets)
  O6  the expert-grouped order of the flat assignments a = t*k + j, stable in t
  O7  per expert: G = X W_gu^T, h = gelu_tanh(G[:, :I]) * G[:, I:], Y = h W_d^T
  O8  out[t] = sum_j w[t, j] * Y[inv[t*k + j]]
  O9  MXFP4 expert weights decoded to fp64 before O7
  O11 W4A4 (MXFP4 weights and activations): x, and the bf16 h of every GEGLU,
      are quantised per 32 consecutive K values to MXFP4 (the OCP MX v1.0
      conversion: shared scale 2^(floor(log2 amax) - 2), elements rounded to
      the nearest E2M1 value, ties to the even code, saturating at 6) before
      their matmuls; the router keeps the bf16 x (the pages name w4a4 MXFP4
      checkpoints: vLLM-Ascend Gemma4 tutorial, section 3.1)
  O12 NVFP4 expert weights (the format of the Gemma-4-26B-A4B-NVFP4
      checkpoint of the verification report) decoded to fp64 before O7:
      E2M1 element x FP8 E4M3 scale of its 16-element block x the matrix's
      fp32 scale
  O13 NVFP4 weights and activations (nv_a4): x, and the bf16 h of every
      GEGLU, are quantised per 16 consecutive K values to NVFP4 before their
      matmuls (the verification report's quantisation table, section 2.3,
      gives 4-bit float with group size 16 for weights and activations):
      relative to the tensor's fp32 input scale g, a block's E4M3 scale is
      the nearest E4M3 value to amax / (6 g) (ties to the even code,
      saturating at 448), and each value v / (scale g) goes to the nearest
      E2M1 value (ties to the even code, saturating at 6); these decisions
      are taken in fp32, as a kernel takes them
  O10 shapes with a dense MLP (I_sh > 0): out[t] += MLP(x[t]) with
      MLP(x) = (gelu_tanh(x Wg^T) * (x Wu^T)) Wd^T, the same GEGLU form as an
      expert, weight 1 (the block runs its dense MLP of intermediate 2112 next
      to the MoE: optimisation report, section 1; the two outputs being
      summed is this repository's reading, the pages do not spell it out)

Readings of points the pages leave open (renormalised top-k softmax,
lowest-index tie-break, gate = first I rows of the concatenated gate/up
weight, the tanh GELU constants, no capacity limit) are listed with the
design notes of the repository.

Parity status: O2-O8 are pinned by the dense brute force (`dense_forward`) and
by closed-form special cases in the CPU test suite; O9 is pinned by the E2M1
table of the OCP Microscaling Formats v1.0 specification; O12's E4M3 table by
torch's float8_e4m3fn decoding of all finite codes; O13's E4M3 rounding by
torch's float8_e4m3fn cast at every midpoint and by the generator's own
encoder, its block rule by a per-value scalar rule, and a one-expert layer by
a textbook torch GEGLU FFN on the quantised operands.  Against the real
Gemma-4 layer parity is unpinned: the pages print no activations or weights.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64", "mxfp4_to_f64", "router_logits", "topk_softmax",
    "counts_offsets", "permutation", "gelu_tanh", "gateup_geglu",
    "down_proj", "combine", "expert_weights", "forward", "forward_tokens",
    "dense_forward", "routing_margin", "shared_weights", "shared_mlp",
    "mx_quantize", "mx_dequantize", "mx_round", "round_to_bf16",
    "e4m3_to_f64", "nvfp4_to_f64", "e4m3_nearest", "nv_quantize", "nv_dequantize", "nv_round",
]


# ---------------------------------------------------------------- O1 / O9
def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64 (O1)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# FP4 E2M1 element values by code (OCP Microscaling Formats v1.0): bit 3 is
# the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa; code 1 is
# the subnormal 0.5.
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                  -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def mxfp4_to_f64(packed, scales) -> np.ndarray:
    """Decode MXFP4 weights to fp64 (O9).

    packed [..., K/2] holds two E2M1 codes per byte, the even K index in the
    low nibble; scales [..., K/32] holds one E8M0 byte per 32 consecutive K
    elements, meaning 2^(byte - 127).  MXFP4 checkpoints of this model are
    named by the vLLM-Ascend Gemma4 tutorial (section 3.1 model weight); the
    element and scale encodings are those of the OCP MX v1.0 specification.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    vals = _E2M1[codes]
    s = np.asarray(scales, dtype=np.int64)
    if np.any(s == 255):
        raise ValueError("E8M0 byte 0xFF is NaN and not a valid scale")
    factor = np.ldexp(1.0, s - 127)                     # [..., K/32]
    K = codes.shape[-1]
    vals = vals.reshape(*codes.shape[:-1], K // 32, 32) * factor[..., None]
    return vals.reshape(*codes.shape[:-1], K)


# ---------------------------------------------------------------- O12
def _e4m3_table() -> np.ndarray:
    """Values of the 256 FP8 E4M3 codes (OCP 8-bit floating point
    specification, E4M3: sign bit, four exponent bits with bias 7, three
    mantissa bits; exponent field 0 is subnormal, 2^-6 * m/8; no
    infinities; S.1111.111 is NaN, so 448 is the largest finite value)."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        ef, m = (c >> 3) & 0xF, c & 0x7
        if ef == 0xF and m == 0x7:
            t[c] = np.nan
        elif ef == 0:
            t[c] = sign * math.ldexp(m / 8.0, -6)
        else:
            t[c] = sign * math.ldexp(1.0 + m / 8.0, ef - 7)
    return t


_E4M3 = _e4m3_table()


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact values of FP8 E4M3 codes (O12)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def nvfp4_to_f64(packed, scales, glob) -> np.ndarray:
    """Decode one NVFP4 matrix to fp64 (O12).

    packed [..., K/2] holds two E2M1 codes per byte, the even K index in the
    low nibble (as for MXFP4); scales [..., K/16] one E4M3 code per 16
    consecutive K elements; glob the matrix's fp32 scale.  Element value =
    E2M1(code) * E4M3(scale) * glob."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.stack([packed & 0x0F, packed >> 4], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    K = codes.shape[-1]
    sc = e4m3_to_f64(scales)
    if np.any(np.isnan(sc)):
        raise ValueError("E4M3 NaN code used as a scale")
    vals = _E2M1[codes].reshape(*codes.shape[:-1], K // 16, 16) * sc[..., None]
    return vals.reshape(*codes.shape[:-1], K) * float(np.float32(glob))


# ---------------------------------------------------------------- O13
def e4m3_nearest(v) -> np.ndarray:
    """Code of the E4M3 value nearest to each non-negative v (O13): the
    least distance over the 127 finite non-negative codes, the even code on
    a tie (round half to even), 448 (code 0x7E) for everything from 448 up."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("E4M3 scales are taken of non-negative amax values")
    grid = _E4M3[:127]                                   # codes 0x00 .. 0x7E, ascending values
    dist = np.abs(v[..., None] - grid)                   # [..., 127]
    best = dist.min(axis=-1, keepdims=True)
    score = np.where(dist == best, np.arange(127) % 2, 2)   # even codes first on a tie
    code = np.argmin(score, axis=-1)
    return np.where(v >= 448.0, 0x7E, code).astype(np.uint8)


def nv_quantize(v, g):
    """NVFP4 codes of rows of values, per 16 along the last axis, relative to
    the tensor's fp32 scale g (O13).  Returns (codes uint8 [..., K], one
    E2M1 code per value, and E4M3 block-scale codes uint8 [..., K/16]).

    In fp32, as a kernel computes them: amax of the block, s = amax / (6 g)
    (6 g rounded to fp32 first), its E4M3 code; then step = scale * g and
    each value's quotient v / step, both rounded to fp32, whose nearest E2M1
    code (ties to the even code, saturating at 6, the sign kept) is the
    value's code.  A block whose scale code is 0 gets all-zero codes."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % 16:
        raise ValueError("NVFP4 blocks need K % 16 == 0")
    v32 = v.astype(np.float32)
    if not np.array_equal(v32.astype(np.float64), v):
        raise ValueError("NVFP4 activations must be fp32 values (here: bf16)")
    g32 = np.float32(g)
    blk = v32.reshape(*v.shape[:-1], K // 16, 16)
    amax = np.max(np.abs(blk), axis=-1)
    with np.errstate(over="ignore"):
        s = amax / (np.float32(6.0) * g32)                 # float32 arithmetic
    sc = e4m3_nearest(s.astype(np.float64))
    step = (e4m3_to_f64(sc).astype(np.float32) * g32)    # float32
    safe = np.where(step > 0, step, np.float32(1.0))
    q = (blk / safe[..., None]).astype(np.float64)       # float32 quotient, widened exactly
    dist = np.abs(np.abs(q)[..., None] - np.asarray(_E2M1_MAG))
    best = dist.min(axis=-1, keepdims=True)
    score = np.where(dist == best, np.where(np.arange(8) % 2 == 0, 0, 1), 2)
    code = np.argmin(score, axis=-1).astype(np.uint8) | np.where(np.signbit(q), 8, 0).astype(np.uint8)
    code = np.where((step > 0)[..., None], code, 0).astype(np.uint8)
    return code.reshape(v.shape), sc


def nv_dequantize(codes, scales, g) -> np.ndarray:
    """Values of one-code-per-value NVFP4 data: E2M1 x E4M3 block scale x g."""
    codes = np.asarray(codes, dtype=np.int64)
    K = codes.shape[-1]
    vals = _E2M1[codes].reshape(*codes.shape[:-1], K // 16, 16) * e4m3_to_f64(scales)[..., None]
    return vals.reshape(codes.shape) * float(np.float32(g))


def nv_round(v, g) -> np.ndarray:
    """v quantised to NVFP4 relative to the scale g and decoded again."""
    return nv_dequantize(*nv_quantize(v, g), g)


def expert_weights(inp, e: int):
    """fp64 gate/up [2I, H] and down [H, I] weights of expert e."""
    if getattr(inp.shape, "nvfp4", False):
        wgu = nvfp4_to_f64(inp.w_gate_up[e], inp.gu_scales[e], inp.gu_global[e])
        wd = nvfp4_to_f64(inp.w_down[e], inp.d_scales[e], inp.d_global[e])
        return wgu, wd
    if inp.shape.mxfp4:
        wgu = mxfp4_to_f64(inp.w_gate_up[e], inp.gu_scales[e])
        wd = mxfp4_to_f64(inp.w_down[e], inp.d_scales[e])
    else:
        wgu = bf16_to_f64(inp.w_gate_up[e])
        wd = bf16_to_f64(inp.w_down[e])
    return wgu, wd


# ---------------------------------------------------------------- O11
_E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7, code 8..15 negative


def _e2m1_code(q: float) -> int:
    """Nearest E2M1 code of q (already divided by the block scale): the
    magnitude with the least distance, the even code on a tie, 6 for
    everything beyond; the sign bit from q's sign (so -0.0 -> code 8)."""
    m = abs(q)
    best = 0
    for c in range(1, 8):
        d, db = abs(m - _E2M1_MAG[c]), abs(m - _E2M1_MAG[best])
        if d < db or (d == db and c % 2 == 0):
            best = c
    return best | (8 if math.copysign(1.0, q) < 0 else 0)


def mx_quantize(v) -> tuple:
    """MXFP4 codes and E8M0 scale bytes of rows of values, per 32 along the
    last axis (O11).  Returns (codes uint8 [..., K] one code per value,
    scales uint8 [..., K/32]).  A block's scale exponent is floor(log2 amax)
    - 2, clamped to [-127, 127]; an all-zero block gets exponent 0.  Each
    value takes the grid magnitude at the least distance (an array of all
    eight distances), the even code on a tie, and its own sign bit -- the
    rule of `_e2m1_code`, which the tests compare this against."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % 32:
        raise ValueError("MXFP4 blocks need K % 32 == 0")
    blk = v.reshape(*v.shape[:-1], K // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    ex = np.frexp(amax)[1].astype(np.int64) - 1 - 2          # floor(log2 amax) - 2
    e = np.where(amax == 0.0, 0, np.clip(ex, -127, 127))
    q = blk / np.ldexp(1.0, e)[..., None]                     # exact: a power of two
    dist = np.abs(np.abs(q)[..., None] - np.asarray(_E2M1_MAG))    # [..., 32, 8]
    best = dist.min(axis=-1, keepdims=True)
    tie_pref = np.where(np.arange(8) % 2 == 0, 0, 1)          # even codes first on a tie
    score = np.where(dist == best, tie_pref, 2)
    code = np.argmin(score, axis=-1).astype(np.uint8)
    code = code | np.where(np.signbit(q), 8, 0).astype(np.uint8)
    return code.reshape(v.shape), (e + 127).astype(np.uint8)


def mx_dequantize(codes, scales) -> np.ndarray:
    """Values of one-code-per-value MXFP4 data (O11)."""
    codes = np.asarray(codes, dtype=np.int64)
    K = codes.shape[-1]
    vals = _E2M1[codes].reshape(*codes.shape[:-1], K // 32, 32)
    f = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (vals * f[..., None]).reshape(codes.shape)


def mx_round(v) -> np.ndarray:
    """v quantised to MXFP4 and decoded again."""
    return mx_dequantize(*mx_quantize(v))


def round_to_bf16(v) -> np.ndarray:
    """fp64 -> fp32 (nearest even) -> bf16 (nearest even), as an fp32 kernel
    rounds a value it holds in fp32."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def shared_weights(inp):
    """fp64 gate/up [2 I_sh, H] and down [H, I_sh] of the dense MLP (O10), or
    None when the shape has none."""
    if inp.shape.I_sh <= 0:
        return None
    if inp.shape.mxfp4:
        return (mxfp4_to_f64(inp.w_sh_gate_up, inp.sh_gu_scales),
                mxfp4_to_f64(inp.w_sh_down, inp.sh_d_scales))
    return bf16_to_f64(inp.w_sh_gate_up), bf16_to_f64(inp.w_sh_down)


# ---------------------------------------------------------------- O2
def router_logits(x64: np.ndarray, wr64: np.ndarray, bias=None) -> np.ndarray:
    """L[t, e] = sum_h x[t, h] W_r[e, h] (+ b[e]) in fp64 (O2).

    The router linear layer ahead of the fused gating op (optimisation report,
    section 5, MoE Router row)."""
    L = x64 @ wr64.T
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


# ---------------------------------------------------------------- O3 / O4
def topk_softmax(L: np.ndarray, k: int):
    """Top-k selection and renormalised softmax weights (O3, O4).

    For each token the experts are ordered by the key (-L[t, e], e): largest
    logit first, the lower expert index first among equal logits.  The first
    k are the selection, in slot order.  w[t, j] = exp(L_j - L_0) / sum over
    the k selected of exp(L_i - L_0), which equals the softmax over all
    experts renormalised over the selected ones (optimisation report, section
    5: the router is fused as a gating top-k softmax op).

    Returns ids int32 [T, k], w float64 [T, k]."""
    L = np.asarray(L, dtype=np.float64)
    T, E = L.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -L[t]))     # primary -L, then index
        sel = order[:k]
        ids[t] = sel
        z = L[t, sel] - L[t, sel[0]]
        ez = np.exp(z)
        w[t] = ez / ez.sum()
    return ids, w


def routing_margin(L: np.ndarray, k: int) -> np.ndarray:
    """Per token, the gap between the k-th and (k+1)-th largest logit
    (infinite when k equals the expert count)."""
    L = np.asarray(L, dtype=np.float64)
    if k >= L.shape[1]:
        return np.full(L.shape[0], np.inf)
    s = -np.sort(-L, axis=1)
    return s[:, k - 1] - s[:, k]


# ---------------------------------------------------------------- O5 / O6
def counts_offsets(ids: np.ndarray, E: int):
    """counts[e] = number of (t, j) with ids[t, j] == e; offsets = exclusive
    prefix sum with offsets[E] = T*k (O5).  These are the data-dependent split
    sizes of the dispatch (optimisation report, section 6.1)."""
    flat = np.asarray(ids).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[int(e)] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    return counts.astype(np.int32), offsets.astype(np.int32)


def permutation(ids: np.ndarray):
    """Expert-grouped order of the flat assignments (O6).

    sorted_ids[p] = a = t*k + j, ordered by (ids[t, j], t); a token never
    picks an expert twice, so the order is unique.  inv[a] = p."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    tok = np.arange(T * k) // k
    sorted_ids = np.lexsort((tok, flat)).astype(np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    inv[sorted_ids] = np.arange(T * k, dtype=np.int32)
    return sorted_ids, inv


# ---------------------------------------------------------------- O7
_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)


def gelu_tanh(z):
    """gelu_pytorch_tanh (verification report, section 2.1): the tanh form of
    the Gaussian error linear unit of Hendrycks and Gimpel,
    0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(_SQRT_2_OVER_PI * (z + 0.044715 * z ** 3)))


def gateup_geglu(X: np.ndarray, wgu64: np.ndarray) -> np.ndarray:
    """h = gelu_tanh(X W_gate^T) * (X W_up^T) for one expert (O7, first half).

    wgu64 is [2I, H]: rows 0..I-1 the gate, rows I..2I-1 the up projection
    (the GEGLU of the optimisation report, section 1)."""
    I = wgu64.shape[0] // 2
    G = X @ wgu64.T
    return gelu_tanh(G[:, :I]) * G[:, I:]


def down_proj(h: np.ndarray, wd64: np.ndarray) -> np.ndarray:
    """Y = h W_d^T for one expert, W_d [H, I] (O7, second half)."""
    return h @ wd64.T


def shared_mlp(X: np.ndarray, wsh, a4: bool = False) -> np.ndarray:
    """The dense MLP on rows X (O10): the expert GEGLU FFN with the dense
    weights (and, under W4A4, its h quantised like an expert's); zeros when
    wsh is None."""
    if wsh is None:
        return np.zeros_like(X)
    h = gateup_geglu(X, wsh[0])
    if a4:
        h = mx_round(round_to_bf16(h))
    return down_proj(h, wsh[1])


# ---------------------------------------------------------------- O8
def combine(Y: np.ndarray, inv: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] Y[inv[t*k + j]] (O8): the weighted sum of each
    token's expert outputs (the local-expert sum before the all-reduce of the
    decode path, optimisation report, section 6.1)."""
    T, k = w.shape
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * Y[inv[t * k + j]]
    return out


# ---------------------------------------------------------------- whole layer
def _expert_input(inp, x64):
    """The expert matmuls' view of x: itself, or quantised (O11 MXFP4, O13
    NVFP4 relative to the gate/up input scale)."""
    if getattr(inp.shape, "nv_a4", False):
        return nv_round(x64, inp.gu_input_scale)
    return mx_round(x64) if getattr(inp.shape, "a4", False) else x64


def _down_input(inp, h):
    """The down matmul's view of an expert's h: h, or its bf16 rounding
    quantised (O11 MXFP4, O13 NVFP4 relative to the down input scale)."""
    if getattr(inp.shape, "nv_a4", False):
        return nv_round(round_to_bf16(h), inp.d_input_scale)
    return mx_round(round_to_bf16(h)) if getattr(inp.shape, "a4", False) else h


def forward(inp, logits_fp32: np.ndarray | None = None) -> dict:
    """The routed layer, step by step (O1-O9).

    If logits_fp32 is given, routing uses those float32 values (widened
    exactly) instead of O2; this is how the routing decision is taken in the
    same precision as a float32 kernel."""
    s = inp.shape
    T, H, E, k, I = s.T, s.H, s.E, s.k, s.I
    x64 = bf16_to_f64(inp.x)
    L = router_logits(x64, bf16_to_f64(inp.w_router), inp.router_bias)
    Lr = L if logits_fp32 is None else np.asarray(logits_fp32, dtype=np.float32).astype(np.float64)
    ids, w = topk_softmax(Lr, k)
    counts, offsets = counts_offsets(ids, E)
    sorted_ids, inv = permutation(ids)
    a4 = getattr(s, "a4", False)
    xe = _expert_input(inp, x64)          # what the expert matmuls read (O11, O13)
    Y = np.zeros((T * k, H), dtype=np.float64)
    Hh = np.zeros((T * k, I), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue                      # empty expert: its weights are never read
        rows = sorted_ids[lo:hi]
        X = xe[rows // k]
        wgu, wd = expert_weights(inp, e)
        h = _down_input(inp, gateup_geglu(X, wgu))
        Hh[lo:hi] = h
        Y[lo:hi] = down_proj(h, wd)
    out = combine(Y, inv, w) + shared_mlp(xe, shared_weights(inp), a4)
    return dict(logits=L, route_logits=Lr, ids=ids, w=w, counts=counts,
                offsets=offsets, sorted_ids=sorted_ids, inv=inv, h=Hh, y=Y,
                out=out, margin=routing_margin(Lr, k))


def forward_tokens(inp, tokens) -> dict:
    """The layer evaluated one token at a time for the listed tokens (the
    output of a token depends only on its own row).  Used to sample the
    output of large problems."""
    s = inp.shape
    k = s.k
    tokens = np.asarray(tokens, dtype=np.int64)
    x64 = bf16_to_f64(inp.x[tokens])
    L = router_logits(x64, bf16_to_f64(inp.w_router), inp.router_bias)
    ids, w = topk_softmax(L, k)
    a4 = getattr(s, "a4", False)
    xe = _expert_input(inp, x64)
    out = np.zeros((len(tokens), s.H), dtype=np.float64)
    cache = {}
    for i in range(len(tokens)):
        for j in range(k):
            e = int(ids[i, j])
            if e not in cache:
                cache[e] = expert_weights(inp, e)
            wgu, wd = cache[e]
            h = _down_input(inp, gateup_geglu(xe[i:i + 1], wgu))
            out[i] += w[i, j] * down_proj(h, wd)[0]
    out += shared_mlp(xe, shared_weights(inp), a4)
    return dict(logits=L, ids=ids, w=w, out=out, margin=routing_margin(L, k))


def dense_forward(inp) -> np.ndarray:
    """Brute force: every expert on every token, masked to the top-k.

    mask[t, e] = 1 iff fewer than k experts e' beat e, where e' beats e when
    L[t, e'] > L[t, e], or L[t, e'] == L[t, e] and e' < e (a rank count that
    does not sort).  out[t] = sum_e mask * p_hat * F_e(x_t), p_hat the softmax
    over the masked set.  Only for small problems."""
    s = inp.shape
    T, E, k = s.T, s.E, s.k
    x64 = bf16_to_f64(inp.x)
    L = router_logits(x64, bf16_to_f64(inp.w_router), inp.router_bias)
    mask = np.zeros((T, E), dtype=bool)
    for t in range(T):
        for e in range(E):
            beats = 0
            for e2 in range(E):
                if L[t, e2] > L[t, e] or (L[t, e2] == L[t, e] and e2 < e):
                    beats += 1
            mask[t, e] = beats < k
    out = np.zeros((T, s.H), dtype=np.float64)
    for t in range(T):
        m = max(L[t, e] for e in range(E) if mask[t, e])
        den = sum(math.exp(L[t, e] - m) for e in range(E) if mask[t, e])
        for e in range(E):
            if not mask[t, e]:
                continue
            wgu, wd = expert_weights(inp, e)
            F = down_proj(gateup_geglu(x64[t:t + 1], wgu), wd)[0]
            out[t] += (math.exp(L[t, e] - m) / den) * F
    return out + shared_mlp(x64, shared_weights(inp))
