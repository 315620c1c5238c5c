"""GPU parity of the grouped expert GEMMs and the combine, each fed the same
inputs as the oracle: gate/up + GEGLU (gathered and pre-permuted rows, bf16
and MXFP4 weights), down, and the weighted combine."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, REL_L2

pytestmark = pytest.mark.gpu


def _ids_with_ragged_counts(T, E, k, seed):
    """Routing with a Zipf-like popularity so counts are ragged and some
    experts may be empty."""
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    return mi.random_ids(T, E, k, seed=seed, p=p / p.sum())


def _setup(T, H, E, k, I, mx, seed):
    inp = mi.make(mi.Shape(T=T, H=H, E=E, k=k, I=I, mxfp4=mx), seed=seed)
    ids = _ids_with_ragged_counts(T, E, k, seed)
    counts, offsets = oracle.counts_offsets(ids, E)
    sorted_ids, inv = oracle.permutation(ids)
    return inp, ids, counts, offsets, sorted_ids, inv


def _errs(got, ref):
    d = got - ref
    return np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300), float(np.abs(d).max())


U32 = 2.0 ** -24     # fp32 unit roundoff
U16 = 2.0 ** -8      # bf16 unit roundoff (8 significant bits)


def _acc_err(absdot, K):
    """Bound on the fp32 accumulation error of a K-long dot product summed in
    MFMA steps of 32 products: at most K/32 + 32 roundings, each of a partial
    sum no larger than sum |a b|."""
    return (K / 32 + 32) * U32 * absdot


# Cases span several row blocks and a ragged tail, and hit the three row-block
# sizes (16 rows up to a mean of 16 rows per expert, 64 up to 40, 256 above).
CASES = [
    (64, 512, 16, 2, 192),     # mean 8 rows/expert
    (300, 512, 16, 2, 192),    # mean 37: 64-row tiles
    (300, 512, 16, 4, 192),    # mean 75: 256-row tiles
    (1000, 256, 8, 2, 128),    # mean 250
    (257, 2816, 128, 8, 704),  # Gemma-4 expert shape, mean 16
    (4096, 512, 128, 8, 256),  # mean 256: 512 down tiles of 256 rows, two rounds per CU
    (1000, 320, 8, 2, 192),    # mean 250, 256-row tiles: last down column tile 64 of 256 wide, last gate/up one half
    # the prefill tile (256 x 256, sixteen waves; bf16: two token and three
    # weight stages with spread weight loads; MXFP4: codes and scale rows
    # straight to LDS) at the Gemma-4 expert shape, K = 2816 / 704
    (2048, 2816, 128, 8, 704), # the prefill batch: mean 128, single-tile experts stream, hot ones span many tiles
    (1024, 2816, 16, 4, 704),  # mean 256
]


@pytest.mark.parametrize("mx", [False, True], ids=["bf16", "mxfp4"])
@pytest.mark.parametrize("T,H,E,k,I", CASES)
def test_gateup_geglu(gpu, T, H, E, k, I, mx):
    say(f"gateup T={T} H={H} E={E} k={k} I={I} mxfp4={mx}")
    inp, ids, counts, offsets, sorted_ids, inv = _setup(T, H, E, k, I, mx, seed=T + I)
    A = T * k
    s = moe.shape(T, H, E, k, I, mxfp4=mx)
    x = dev.to_device(inp.x)
    w = dev.to_device(inp.w_gate_up)
    sc = dev.to_device(inp.gu_scales) if mx else None
    off = torch.from_numpy(offsets).cuda()
    si = torch.from_numpy(sorted_ids).cuda()
    h = torch.full((A, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu.gemm_gateup(s, x, si, off, w, sc, h)
    # the same with the rows already permuted (x_perm) must match bitwise
    xp = dev.to_device(inp.x[sorted_ids // k])
    h2 = torch.empty_like(h)
    gpu.gemm_gateup(s, xp, None, off, w, sc, h2)
    torch.cuda.synchronize()
    got = h.float().cpu().numpy().astype(np.float64)
    assert (dev.bf16_bits(h) == dev.bf16_bits(h2)).all()
    x64 = oracle.bf16_to_f64(inp.x)
    ref = np.zeros((A, I))
    bound = np.zeros((A, I))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            wgu, _ = oracle.expert_weights(inp, e)
            X = x64[sorted_ids[lo:hi] // k]
            ref[lo:hi] = oracle.gateup_geglu(X, wgu)
            # Elementwise bound: accumulation error dG of gate and up, carried
            # through gelu (|gelu'| <= 1.13) and the product, the fp32 GEGLU
            # evaluation (4e-6 relative) and the final bf16 rounding.
            G = X @ wgu.T
            dG = _acc_err(np.abs(X) @ np.abs(wgu).T, H)
            g, u, dg, du = G[:, :I], G[:, I:], dG[:, :I], dG[:, I:]
            gl = np.abs(oracle.gelu_tanh(g))
            prop = 1.13 * dg * (np.abs(u) + du) + gl * du
            bound[lo:hi] = U16 * (np.abs(ref[lo:hi]) + prop) + prop + 4e-6 * gl * np.abs(u) + 1e-30
    rel, mx_err = _errs(got, ref)
    ratio = float((np.abs(got - ref) / bound).max())
    say(f"  counts min {counts.min()} max {counts.max()}: rel_l2 {rel:.3e} max_abs {mx_err:.3e} "
        f"max err/bound {ratio:.3f}")
    assert np.isfinite(got).all()
    assert rel <= REL_L2 and ratio <= 1.0


@pytest.mark.parametrize("mx", [False, True], ids=["bf16", "mxfp4"])
@pytest.mark.parametrize("T,H,E,k,I", CASES)
def test_down(gpu, T, H, E, k, I, mx):
    say(f"down T={T} H={H} E={E} k={k} I={I} mxfp4={mx}")
    inp, ids, counts, offsets, sorted_ids, inv = _setup(T, H, E, k, I, mx, seed=T + I)
    A = T * k
    s = moe.shape(T, H, E, k, I, mxfp4=mx)
    hb = mi.random_bf16((A, I), sigma=0.5, seed=A)
    h = dev.to_device(hb)
    w = dev.to_device(inp.w_down)
    sc = dev.to_device(inp.d_scales) if mx else None
    off = torch.from_numpy(offsets).cuda()
    y = torch.full((A, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu.gemm_down(s, h, off, w, sc, y)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    h64 = oracle.bf16_to_f64(hb)
    ref = np.zeros((A, H))
    bound = np.zeros((A, H))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            _, wd = oracle.expert_weights(inp, e)
            ref[lo:hi] = oracle.down_proj(h64[lo:hi], wd)
            dY = _acc_err(np.abs(h64[lo:hi]) @ np.abs(wd).T, I)
            bound[lo:hi] = U16 * (np.abs(ref[lo:hi]) + dY) + dY + 1e-30
    rel, mx_err = _errs(got, ref)
    ratio = float((np.abs(got - ref) / bound).max())
    say(f"  rel_l2 {rel:.3e} max_abs {mx_err:.3e} max err/bound {ratio:.3f}")
    assert np.isfinite(got).all()
    assert rel <= REL_L2 and ratio <= 1.0


@pytest.mark.parametrize("T,H,I", [(150, 512, 192), (300, 512, 192), (24, 512, 192), (1200, 512, 192),
                                   (1200, 2816, 704)])
def test_mxfp4_equals_bf16_on_dequantised_weights(gpu, T, H, I):
    """MXFP4 decodes exactly to bf16, so the MXFP4 kernels must reproduce the
    bf16 kernels fed the decoded weights, bitwise (E=16, k=4; T=150, mean 37
    rows per expert: 64-row tiles with 64-wide K steps, codes through
    registers; T=24: 16-row tiles, 4-bit gate/up in 256-wide steps against
    bf16 in 128-wide steps; T=300 and T=1200: 256-row tiles, 4-bit codes and
    the tile's scale rows straight to LDS, at K = 512 / 192 and at the
    Gemma-4 expert shape, K = 2816 / 704 -- the MFMAs still run in K order)."""
    E, k = 16, 4
    say(f"mxfp4 vs bf16 T={T} H={H} E={E} k={k} I={I}")
    inp, ids, counts, offsets, sorted_ids, inv = _setup(T, H, E, k, I, True, seed=5)
    A = T * k
    dq_gu = np.stack([oracle.expert_weights(inp, e)[0] for e in range(E)]).astype(np.float32)
    dq_d = np.stack([oracle.expert_weights(inp, e)[1] for e in range(E)]).astype(np.float32)
    bits_gu = (dq_gu.view(np.uint32) >> 16).astype(np.uint16)     # exact: 2 significant bits
    bits_d = (dq_d.view(np.uint32) >> 16).astype(np.uint16)
    assert (mi.bf16_bits_to_f32(bits_gu) == dq_gu).all()
    off = torch.from_numpy(offsets).cuda()
    si = torch.from_numpy(sorted_ids).cuda()
    x = dev.to_device(inp.x)
    s_mx = moe.shape(T, H, E, k, I, mxfp4=True)
    s_bf = moe.shape(T, H, E, k, I)
    h_mx = torch.empty((A, I), dtype=torch.bfloat16, device="cuda")
    h_bf = torch.empty_like(h_mx)
    gpu.gemm_gateup(s_mx, x, si, off, dev.to_device(inp.w_gate_up), dev.to_device(inp.gu_scales), h_mx)
    gpu.gemm_gateup(s_bf, x, si, off, dev.to_device(bits_gu), None, h_bf)
    y_mx = torch.empty((A, H), dtype=torch.bfloat16, device="cuda")
    y_bf = torch.empty_like(y_mx)
    gpu.gemm_down(s_mx, h_bf, off, dev.to_device(inp.w_down), dev.to_device(inp.d_scales), y_mx)
    gpu.gemm_down(s_bf, h_bf, off, dev.to_device(bits_d), None, y_bf)
    torch.cuda.synchronize()
    assert (dev.bf16_bits(h_mx) == dev.bf16_bits(h_bf)).all()
    assert (dev.bf16_bits(y_mx) == dev.bf16_bits(y_bf)).all()


def _cache_groups(counts, H, max_bytes, min_mean):
    """Consecutive expert ranges whose rows' down output (rows x H bf16) fits
    in max_bytes, each with more than min_mean rows per expert."""
    groups, e0, rows = [], 0, 0
    for e, c in enumerate(counts):
        if rows and (rows + c) * H * 2 > max_bytes:
            groups.append((e0, e))
            e0, rows = e, 0
        rows += c
    groups.append((e0, len(counts)))
    for a, b in groups:
        assert counts[a:b].sum() * H * 2 <= max_bytes and counts[a:b].sum() > min_mean * (b - a)
    return groups


def test_down_reversed_group_order(gpu):
    """8192 Zipf-routed tokens at the Gemma-4 expert shape: the down GEMM's
    output (A x H bf16 = 369 MB) exceeds the 256 MB last-level cache, so each
    XCD runs its row-tile groups last to first.  The whole output is checked
    against the oracle's elementwise bound, and -- tile arithmetic does not
    depend on the order tiles run in -- bitwise against forward-order calls
    on consecutive expert ranges (offsets rebased, outputs under the cache
    size, still more than 40 rows per expert so the same 256-row tile runs)."""
    T, H, E, k, I = 8192, 2816, 128, 8, 704
    say(f"down reversed order T={T} H={H} E={E} k={k} I={I}")
    inp, ids, counts, offsets, sorted_ids, inv = _setup(T, H, E, k, I, False, seed=11)
    A = T * k
    assert A * H * 2 > 256 << 20
    hb = mi.random_bf16((A, I), sigma=0.5, seed=A + 1)
    h = dev.to_device(hb)
    w = dev.to_device(inp.w_down)
    off = torch.from_numpy(offsets).cuda()
    y = torch.empty((A, H), dtype=torch.bfloat16, device="cuda")
    gpu.gemm_down(moe.shape(T, H, E, k, I), h, off, w, None, y)
    groups = _cache_groups(counts, H, 240 << 20, 40)
    say(f"  counts min {counts.min()} max {counts.max()}; {len(groups)} forward-order expert ranges")
    y_parts = torch.empty_like(y)
    for e0, e1 in groups:
        lo, hi = int(offsets[e0]), int(offsets[e1])
        sub_off = torch.from_numpy((offsets[e0:e1 + 1] - lo).astype(np.int32)).cuda()
        gpu.gemm_down(moe.shape(hi - lo, H, e1 - e0, 1, I), h[lo:hi], sub_off, w[e0:e1], None, y_parts[lo:hi])
    torch.cuda.synchronize()
    assert (dev.bf16_bits(y) == dev.bf16_bits(y_parts)).all()
    del y_parts
    got = y.float().cpu().numpy().astype(np.float64)
    del y
    h64 = oracle.bf16_to_f64(hb)
    worst, num, den = 0.0, 0.0, 0.0
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            _, wd = oracle.expert_weights(inp, e)
            ref = oracle.down_proj(h64[lo:hi], wd)
            dY = _acc_err(np.abs(h64[lo:hi]) @ np.abs(wd).T, I)
            bound = U16 * (np.abs(ref) + dY) + dY + 1e-30
            d = got[lo:hi] - ref
            worst = max(worst, float((np.abs(d) / bound).max()))
            num += float((d * d).sum())
            den += float((ref * ref).sum())
    rel = (num / den) ** 0.5
    say(f"  rel_l2 {rel:.3e} max err/bound {worst:.3f}")
    assert np.isfinite(got).all()
    assert rel <= REL_L2 and worst <= 1.0


@pytest.mark.parametrize("T,H,k", [(1, 64, 1), (16, 256, 2), (300, 2816, 8), (2048, 2816, 8)])
def test_combine(gpu, T, H, k):
    say(f"combine T={T} H={H} k={k}")
    A = T * k
    E = max(k, 16)
    ids = mi.random_ids(T, E, k, seed=T)
    _, inv = oracle.permutation(ids)
    yb = mi.random_bf16((A, H), sigma=0.3, seed=H + T)
    rng = np.random.default_rng(T)
    wts = rng.random((T, k)).astype(np.float32)
    wts /= wts.sum(axis=1, keepdims=True)
    s = moe.shape(T, H, E, k, 64)
    y = dev.to_device(yb)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out)
    invt = torch.from_numpy(inv).cuda()
    wt = torch.from_numpy(wts).cuda()
    gpu.combine(s, y, invt, wt, out)
    gpu.combine(s, y, invt, wt, out2)
    torch.cuda.synchronize()
    ref = oracle.combine(oracle.bf16_to_f64(yb), inv, wts.astype(np.float64))
    got = out.float().cpu().numpy().astype(np.float64)
    # fp32 sum of k terms then one bf16 rounding: |err| <= 2^-8 |ref| + k 2^-23 sum|w y|
    bound = 2.0 ** -8 * np.abs(ref) + k * 2.0 ** -23 * oracle.combine(
        np.abs(oracle.bf16_to_f64(yb)), inv, wts.astype(np.float64)) + 1e-30
    assert (np.abs(got - ref) <= bound).all()
    assert (dev.bf16_bits(out) == dev.bf16_bits(out2)).all()


@pytest.mark.parametrize("T", [150, 300, 24])
def test_nvfp4_equals_bf16_on_dequantised_weights(gpu, T):
    """With every expert's fp32 scale 1, NVFP4 weights decode exactly to bf16
    (E2M1 x E4M3), so the NVFP4 kernels must reproduce the bf16 kernels fed
    the decoded weights, bitwise."""
    H, E, k, I = 512, 16, 4, 192
    inp = mi.make(mi.Shape(T=T, H=H, E=E, k=k, I=I, nvfp4=True), seed=6)
    ids = _ids_with_ragged_counts(T, E, k, 6)
    counts, offsets = oracle.counts_offsets(ids, E)
    sorted_ids, inv = oracle.permutation(ids)
    A = T * k
    ones = np.ones(E, dtype=np.float32)
    dq_gu = np.stack([oracle.nvfp4_to_f64(inp.w_gate_up[e], inp.gu_scales[e], 1.0) for e in range(E)])
    dq_d = np.stack([oracle.nvfp4_to_f64(inp.w_down[e], inp.d_scales[e], 1.0) for e in range(E)])
    bits_gu = mi.f32_to_bf16_bits(dq_gu.astype(np.float32))
    bits_d = mi.f32_to_bf16_bits(dq_d.astype(np.float32))
    assert (mi.bf16_bits_to_f32(bits_gu) == dq_gu).all() and (mi.bf16_bits_to_f32(bits_d) == dq_d).all()
    off = torch.from_numpy(offsets).cuda()
    si = torch.from_numpy(sorted_ids).cuda()
    x = dev.to_device(inp.x)
    s_nv = moe.shape(T, H, E, k, I, nvfp4=True)
    s_bf = moe.shape(T, H, E, k, I)
    h_nv = torch.empty((A, I), dtype=torch.bfloat16, device="cuda")
    h_bf = torch.empty_like(h_nv)
    gpu.gemm_gateup(s_nv, x, si, off, dev.to_device(inp.w_gate_up),
                    dev.to_device(moe.nvfp4_scale_buffer(ones, inp.gu_scales)), h_nv)
    gpu.gemm_gateup(s_bf, x, si, off, dev.to_device(bits_gu), None, h_bf)
    y_nv = torch.empty((A, H), dtype=torch.bfloat16, device="cuda")
    y_bf = torch.empty_like(y_nv)
    gpu.gemm_down(s_nv, h_bf, off, dev.to_device(inp.w_down),
                  dev.to_device(moe.nvfp4_scale_buffer(ones, inp.d_scales)), y_nv)
    gpu.gemm_down(s_bf, h_bf, off, dev.to_device(bits_d), None, y_bf)
    torch.cuda.synchronize()
    assert (dev.bf16_bits(h_nv) == dev.bf16_bits(h_bf)).all()
    assert (dev.bf16_bits(y_nv) == dev.bf16_bits(y_bf)).all()
