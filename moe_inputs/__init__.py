"""Seeded synthetic inputs for the MoE FFN layer (router -> top-k -> dispatch ->
grouped GEGLU experts -> combine).

This module draws random numbers and stores them in the byte formats both
sides consume; it holds none of the layer's arithmetic.  The oracle and the
HIP path both read what it returns.

Shapes follow the Gemma-4-26B-A4B MoE FFN: hidden 2816 (Gemma-4-26B-A4B-NVFP4
Ascend verification report, section 2.1 model architecture parameters), 128
experts with top-8 routing and expert intermediate 704 with a GEGLU activation
(Gemma-4-26B-A4B optimisation report, section 1 model overview).  The pages
print no data for the layer, so every value here is synthetic:

* generator: ``numpy.random.default_rng(seed)`` (PCG64), float32
  ``standard_normal`` draws, in the order router weight, gate/up weight expert
  by expert, down weight expert by expert, then x;
* weights are scaled by sigma = 0.02 and x by 1.0 (float32 multiply), then
  rounded to bfloat16 with round-to-nearest-even;
* skewed routing adds a router bias b_e = ln p_e with p following Zipf(1.2)
  over the expert rank r = e + 1;
* MXFP4 experts quantise the bf16 expert weights per 32-element block along K
  with the OCP Microscaling Formats v1.0 conversion (shared E8M0 scale
  2^(floor(log2 amax) - 2), elements rounded to nearest-even E2M1 and
  saturated at +-6), two codes per byte, low nibble = even K index;
* NVFP4 experts (the format of the Gemma-4-26B-A4B-NVFP4 checkpoint the
  verification report runs) store E2M1 codes like MXFP4 with one FP8 E4M3
  scale per 16 consecutive K elements and one fp32 scale per expert matrix.
  Their synthetic values come from the same bf16 weights: the expert scale is
  amax / (6 * 448) (so the largest block scale lands on the largest E4M3
  value), each block scale is the block's amax / (6 * expert scale) rounded
  to the nearest E4M3 value (ties to the even code, saturating at 448), and
  each element is w / (block scale * expert scale) rounded to the nearest
  E2M1 value as above.

Weight storage is K-contiguous: router [E, H], gate/up [E, 2I, H] with rows
0..I-1 the gate and I..2I-1 the up projection, down [E, H, I].

Shapes with ``I_sh > 0`` add the dense GEGLU MLP that runs next to the MoE in
every decoder block (optimisation report, section 1: intermediate 2112):
gate/up [2 I_sh, H] and down [H, I_sh], drawn like the expert weights
(sigma 0.02, bf16) from their own generator ``default_rng([seed, 2112])`` so
that every other draw is unchanged, and quantised to MXFP4 like the experts
when the experts are.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Shape", "CONFIGS", "make", "make_shape", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "mxfp4_quantize", "nvfp4_quantize", "e4m3_encode",
    "random_bf16", "random_ids",
]


@dataclass(frozen=True)
class Shape:
    """Problem size of one MoE FFN call."""
    T: int          # tokens
    H: int          # hidden size
    E: int          # experts
    k: int          # experts per token
    I: int          # expert intermediate size (gate and up each have I rows)
    skew: bool = False      # add the Zipf(1.2) log-prior router bias
    mxfp4: bool = False     # expert weights stored as MXFP4
    zipf_s: float = 1.2
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    I_sh: int = 0           # intermediate size of the always-on dense MLP (0: none)
    a4: bool = False        # with mxfp4: activations quantised to MXFP4 too (W4A4)
    nvfp4: bool = False     # expert weights stored as NVFP4 (E2M1, E4M3 per 16, fp32 per expert)
    nv_a4: bool = False     # with nvfp4: activations quantised to NVFP4 too (NVFP4 W4A4)

    @property
    def A(self) -> int:
        """Number of (token, slot) assignments, T * k."""
        return self.T * self.k


# The five workloads: a tiny case, then the Gemma-4-26B-A4B layer at decode
# (BS8) and prefill (BS8 x seq 256) sizes, a skewed-routing long prefill and
# the prefill with MXFP4 expert weights.
CONFIGS = {
    "tiny": Shape(T=16, H=256, E=8, k=2, I=128),
    "decode": Shape(T=8, H=2816, E=128, k=8, I=704),
    "prefill": Shape(T=2048, H=2816, E=128, k=8, I=704),
    "skew": Shape(T=8192, H=2816, E=128, k=8, I=704, skew=True),
    "mxfp4": Shape(T=2048, H=2816, E=128, k=8, I=704, mxfp4=True),
    # the decode layer with the block's dense MLP (intermediate 2112) as an
    # always-on shared expert
    "decode_shared": Shape(T=8, H=2816, E=128, k=8, I=704, I_sh=2112),
    # the prefill with MXFP4 experts and MXFP4 activations (W4A4)
    "w4a4": Shape(T=2048, H=2816, E=128, k=8, I=704, mxfp4=True, a4=True),
    # the decode layer with MXFP4 / NVFP4 expert weights (bf16 activations)
    "mxfp4_decode": Shape(T=8, H=2816, E=128, k=8, I=704, mxfp4=True),
    "nvfp4_decode": Shape(T=8, H=2816, E=128, k=8, I=704, nvfp4=True),
    # NVFP4 weights and activations (the Gemma-4-26B-A4B-NVFP4 checkpoint's
    # scheme) at decode and prefill sizes
    "nvfp4_a4_decode": Shape(T=8, H=2816, E=128, k=8, I=704, nvfp4=True, nv_a4=True),
    "nvfp4_a4": Shape(T=2048, H=2816, E=128, k=8, I=704, nvfp4=True, nv_a4=True),
}

# Input (activation) scale of the NVFP4 W4A4 matmuls, for x and for h: a
# checkpoint calibrates it as the activation's amax over 6 x 448; here a
# fixed 2^-8 stands in (E4M3 block scales of amax * 2^8 / 6 stay below 448
# for |values| < 10.5, above the x ~ N(0, 1) and h magnitudes of these
# synthetic layers, and in E4M3's normal range for amax > 0.09).
NV_INPUT_SCALE = np.float32(2.0 ** -8)


def make_shape(name_or_shape) -> Shape:
    if isinstance(name_or_shape, Shape):
        return name_or_shape
    return CONFIGS[name_or_shape]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); uint16 bits.

    NaN inputs are not supported (the generator never draws them)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# E2M1 magnitudes by 3-bit code (OCP Microscaling Formats v1.0, FP4 E2M1):
# exponent bias 1, one mantissa bit, code 1 is the subnormal 0.5.
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _e2m1_encode(q: np.ndarray) -> np.ndarray:
    """Nearest-even E2M1 code of float32 values already divided by the block
    scale, saturating at 6.  Returns uint8 codes 0..15 (bit 3 = sign)."""
    m = np.abs(q)
    # Midpoints between neighbouring grid values; at an exact midpoint the
    # code with an even mantissa bit (even code) wins.
    mids = (_E2M1_GRID[:-1] + _E2M1_GRID[1:]) / 2   # 0.25 .75 1.25 1.75 2.5 3.5 5
    idx = np.searchsorted(mids, m, side="left").astype(np.uint8)  # m <= mid -> lower
    # side="left" gives the lower code at an exact midpoint; where that lower
    # code is odd the tie must go up to the even neighbour.
    lo = np.clip(idx, 0, len(mids) - 1)
    at_mid = (idx < len(mids)) & (m == mids[lo])
    bump = at_mid & ((idx & 1) == 1)
    idx = idx + bump.astype(np.uint8)
    sign = (np.signbit(q)).astype(np.uint8) << np.uint8(3)
    return (idx | sign).astype(np.uint8)


def mxfp4_quantize(w_bits: np.ndarray):
    """Quantise bf16 weights [..., K] (uint16 bits) to MXFP4 along the last axis.

    Returns (packed codes uint8 [..., K/2], scales uint8 [..., K/32]).  K must
    be a multiple of 32.  Blocks whose maximum magnitude is zero get scale
    byte 127 and all-zero codes."""
    w = bf16_bits_to_f32(w_bits)
    K = w.shape[-1]
    if K % 32:
        raise ValueError("MXFP4 needs K % 32 == 0")
    blocks = w.reshape(*w.shape[:-1], K // 32, 32)
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0.0)
    e = np.clip(e, -127, 127).astype(np.int32)
    scale_byte = (e + 127).astype(np.uint8)
    q = blocks / np.ldexp(np.float32(1.0), e)[..., None].astype(np.float32)
    codes = _e2m1_encode(q.astype(np.float32)).reshape(*w.shape[:-1], K)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, scale_byte


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest FP8 E4M3 code (OCP 8-bit floating point: exponent bias 7,
    three mantissa bits, largest finite value 448, no infinities) of
    non-negative values, ties to the even code, saturating at 448."""
    v = np.minimum(np.asarray(v, dtype=np.float64), 448.0)
    out = np.zeros(v.shape, dtype=np.int64)
    pos = v > 0
    e = np.floor(np.log2(np.where(pos, v, 1.0))).astype(np.int64)
    sub = pos & (e < -6)
    # subnormals m * 2^-9 (m = 8 is the smallest normal, code 8, so the
    # codes run on without a seam)
    out = np.where(sub, np.rint(v * 2.0 ** 9).astype(np.int64), out)
    nrm = pos & ~sub
    m = np.rint((v / np.ldexp(1.0, np.where(nrm, e, 0)) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e2 = np.where(carry, e + 1, e)
    m2 = np.where(carry, 0, m)
    out = np.where(nrm, ((e2 + 7) << 3) | m2, out)
    return np.minimum(out, 0x7E).astype(np.uint8)


def _e4m3_value(code: np.ndarray) -> np.ndarray:
    """Value of non-negative E4M3 codes below 0x7F (input preparation only)."""
    c = np.asarray(code, dtype=np.int64)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))


def nvfp4_quantize(w_bits: np.ndarray):
    """Quantise one bf16 weight matrix [..., K] (uint16 bits) to NVFP4 along
    the last axis.  Returns (packed codes uint8 [..., K/2], E4M3 scale codes
    uint8 [..., K/16], the matrix's fp32 scale as a numpy float32).  A block
    whose scale rounds to zero gets all-zero codes."""
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    K = w.shape[-1]
    if K % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    amax = float(np.max(np.abs(w)))
    g = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    blocks = w.reshape(*w.shape[:-1], K // 16, 16)
    bmax = np.max(np.abs(blocks), axis=-1)
    sc = e4m3_encode(bmax / (6.0 * float(g)))
    step = _e4m3_value(sc) * float(g)
    q = np.where(step[..., None] > 0, blocks / np.where(step > 0, step, 1.0)[..., None], 0.0)
    codes = _e2m1_encode(q.astype(np.float32)).reshape(*w.shape[:-1], K)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, sc, g


def zipf_log_prior(E: int, s: float) -> np.ndarray:
    """Router bias b_e = ln p_e with p_r proportional to r^-s, r = e + 1."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


@dataclass
class Inputs:
    shape: Shape
    seed: int
    x: np.ndarray                 # uint16 bf16 bits [T, H]
    w_router: np.ndarray          # uint16 bf16 bits [E, H]
    router_bias: Optional[np.ndarray]   # float32 [E] or None
    w_gate_up: np.ndarray         # uint16 [E, 2I, H], or uint8 packed MXFP4 [E, 2I, H/2]
    w_down: np.ndarray            # uint16 [E, H, I], or uint8 packed MXFP4 [E, H, I/2]
    gu_scales: Optional[np.ndarray] = None   # uint8 [E, 2I, H/32] for MXFP4, E4M3 [E, 2I, H/16] for NVFP4
    d_scales: Optional[np.ndarray] = None    # uint8 [E, H, I/32] for MXFP4, E4M3 [E, H, I/16] for NVFP4
    gu_global: Optional[np.ndarray] = None   # float32 [E]: NVFP4 per-expert scale of gate/up
    d_global: Optional[np.ndarray] = None    # float32 [E]: NVFP4 per-expert scale of down
    # NVFP4 W4A4: the fp32 input scales of the gate/up and down matmuls'
    # activations (calibration constants of the checkpoint; here fixed)
    gu_input_scale: Optional[np.float32] = None
    d_input_scale: Optional[np.float32] = None
    # dense MLP (shape.I_sh > 0): uint16 [2 I_sh, H] and [H, I_sh], or MXFP4
    # codes [2 I_sh, H/2], [H, I_sh/2] with scales [2 I_sh, H/32], [H, I_sh/32]
    w_sh_gate_up: Optional[np.ndarray] = None
    w_sh_down: Optional[np.ndarray] = None
    sh_gu_scales: Optional[np.ndarray] = None
    sh_d_scales: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)


class _Drawer:
    """Draws N(0, sigma^2) float32 values and stores them as bf16 bits,
    reusing its scratch buffers (fresh memory is slow to touch)."""

    def __init__(self, rng):
        self.rng = rng
        self._f = np.empty(0, dtype=np.float32)
        self._u = np.empty(0, dtype=np.uint32)

    def into(self, out: np.ndarray, sigma: float) -> np.ndarray:
        n = out.size
        if self._f.size < n:
            self._f = np.empty(n, dtype=np.float32)
            self._u = np.empty(n, dtype=np.uint32)
        f = self._f[:n]
        self.rng.standard_normal(out=f, dtype=np.float32)
        if sigma != 1.0:
            f *= np.float32(sigma)
        b = f.view(np.uint32)
        u = self._u[:n]
        np.right_shift(b, np.uint32(16), out=u)
        u &= np.uint32(1)
        u += np.uint32(0x7FFF)
        u += b
        np.right_shift(u, np.uint32(16), out=out.reshape(-1), casting="unsafe")
        return out


_WEIGHT_CACHE: dict = {}


def _weights(s: Shape, seed: int):
    """Router and expert weights plus the generator state after drawing them.

    Configurations that differ only in T, skew or the expert format share
    these draws, so they are cached (one copy per (H, E, I, sigma, seed))."""
    key = (s.H, s.E, s.I, s.w_sigma, seed)
    hit = _WEIGHT_CACHE.get(key)
    if hit is not None:
        return hit
    rng = np.random.default_rng(seed)
    d = _Drawer(rng)
    H, E, I = s.H, s.E, s.I
    w_router = d.into(np.empty((E, H), dtype=np.uint16), s.w_sigma)
    w_gu = np.empty((E, 2 * I, H), dtype=np.uint16)
    for e in range(E):
        d.into(w_gu[e], s.w_sigma)
    w_d = np.empty((E, H, I), dtype=np.uint16)
    for e in range(E):
        d.into(w_d[e], s.w_sigma)
    hit = (w_router, w_gu, w_d, rng.bit_generator.state)
    _WEIGHT_CACHE[key] = hit
    return hit


def clear_cache() -> None:
    _WEIGHT_CACHE.clear()
    _MX_CACHE.clear()


_MX_CACHE: dict = {}


def make(config, seed: int = 0) -> Inputs:
    """Draw the inputs of one configuration (a name from CONFIGS or a Shape)."""
    s = make_shape(config)
    if s.a4 and not s.mxfp4:
        raise ValueError("W4A4 (a4) needs MXFP4 weights (mxfp4)")
    if s.nvfp4 and (s.mxfp4 or s.I_sh > 0):
        raise ValueError("NVFP4 experts exclude MXFP4 and the dense MLP")
    if s.nv_a4 and not s.nvfp4:
        raise ValueError("NVFP4 activations (nv_a4) need NVFP4 weights (nvfp4)")
    T, H, E, k, I = s.T, s.H, s.E, s.k, s.I
    w_router, w_gu, w_d, state = _weights(s, seed)
    rng = np.random.default_rng(seed)
    rng.bit_generator.state = state
    x = _Drawer(rng).into(np.empty((T, H), dtype=np.uint16), s.x_sigma)
    bias = zipf_log_prior(E, s.zipf_s) if s.skew else None
    inp = Inputs(shape=s, seed=seed, x=x, w_router=w_router, router_bias=bias,
                 w_gate_up=w_gu, w_down=w_d)
    if s.mxfp4:
        key = (s.H, s.E, s.I, s.w_sigma, seed)
        mx = _MX_CACHE.get(key)
        if mx is None:
            gu_q = np.empty((E, 2 * I, H // 2), dtype=np.uint8)
            gu_s = np.empty((E, 2 * I, H // 32), dtype=np.uint8)
            d_q = np.empty((E, H, I // 2), dtype=np.uint8)
            d_s = np.empty((E, H, I // 32), dtype=np.uint8)
            for e in range(E):
                gu_q[e], gu_s[e] = mxfp4_quantize(w_gu[e])
                d_q[e], d_s[e] = mxfp4_quantize(w_d[e])
            mx = (gu_q, gu_s, d_q, d_s)
            _MX_CACHE[key] = mx
        inp.w_gate_up, inp.gu_scales, inp.w_down, inp.d_scales = mx
    if s.nvfp4:
        key = ("nv", s.H, s.E, s.I, s.w_sigma, seed)
        nv = _MX_CACHE.get(key)
        if nv is None:
            gu_q = np.empty((E, 2 * I, H // 2), dtype=np.uint8)
            gu_s = np.empty((E, 2 * I, H // 16), dtype=np.uint8)
            d_q = np.empty((E, H, I // 2), dtype=np.uint8)
            d_s = np.empty((E, H, I // 16), dtype=np.uint8)
            gu_g = np.empty(E, dtype=np.float32)
            d_g = np.empty(E, dtype=np.float32)
            for e in range(E):
                gu_q[e], gu_s[e], gu_g[e] = nvfp4_quantize(w_gu[e])
                d_q[e], d_s[e], d_g[e] = nvfp4_quantize(w_d[e])
            nv = (gu_q, gu_s, gu_g, d_q, d_s, d_g)
            _MX_CACHE[key] = nv
        inp.w_gate_up, inp.gu_scales, inp.gu_global, inp.w_down, inp.d_scales, inp.d_global = nv
        if s.nv_a4:
            inp.gu_input_scale = inp.d_input_scale = NV_INPUT_SCALE
    if s.I_sh > 0:
        d = _Drawer(np.random.default_rng([seed, 2112]))
        sh_gu = d.into(np.empty((2 * s.I_sh, H), dtype=np.uint16), s.w_sigma)
        sh_d = d.into(np.empty((H, s.I_sh), dtype=np.uint16), s.w_sigma)
        if s.mxfp4:
            inp.w_sh_gate_up, inp.sh_gu_scales = mxfp4_quantize(sh_gu)
            inp.w_sh_down, inp.sh_d_scales = mxfp4_quantize(sh_d)
        else:
            inp.w_sh_gate_up, inp.w_sh_down = sh_gu, sh_d
    return inp


def random_bf16(shape, sigma: float = 1.0, seed: int = 0) -> np.ndarray:
    """bf16 bits of N(0, sigma^2) draws (for step-level tests)."""
    rng = np.random.default_rng(seed)
    return _Drawer(rng).into(np.empty(shape, dtype=np.uint16), sigma)


def random_ids(T: int, E: int, k: int, seed: int = 0, p=None) -> np.ndarray:
    """Random routing table [T, k]: k distinct experts per token, drawn
    without replacement (optionally with popularity p)."""
    rng = np.random.default_rng(seed)
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=k, replace=False, p=p)
    return ids
