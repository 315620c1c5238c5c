"""The seeded input generator: bf16 rounding against torch's conversion,
determinism, the shared-weight prefix property and the skew prior.  CPU only."""
import numpy as np
import torch

import moe_inputs as mi


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        # exact ties: low 16 bits 0x8000 with even and odd bf16 mantissas
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x7F7FFFFF], dtype=np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, -2.5], dtype=np.float32),
    ])
    ours = mi.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    assert (mi.bf16_bits_to_f32(ours) == torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy()).all()


def test_generator_is_deterministic_and_x_is_a_prefix_across_T():
    mi.clear_cache()
    a = mi.make(mi.Shape(T=20, H=64, E=6, k=2, I=32), seed=3)
    mi.clear_cache()
    b = mi.make(mi.Shape(T=7, H=64, E=6, k=2, I=32), seed=3)
    assert (a.x[:7] == b.x).all()
    assert (a.w_gate_up == b.w_gate_up).all() and (a.w_router == b.w_router).all()
    c = mi.make(mi.Shape(T=7, H=64, E=6, k=2, I=32), seed=4)
    assert not (c.x == b.x).all()


def test_weight_statistics():
    a = mi.make(mi.Shape(T=256, H=256, E=8, k=2, I=128), seed=0)
    w = mi.bf16_bits_to_f32(a.w_gate_up)
    x = mi.bf16_bits_to_f32(a.x)
    assert abs(w.std() - 0.02) < 0.001 and abs(x.std() - 1.0) < 0.02


def test_zipf_prior():
    b = mi.zipf_log_prior(128, 1.2).astype(np.float64)
    p = np.exp(b)
    assert abs(p.sum() - 1) < 1e-6
    r = np.arange(1, 129)
    assert np.allclose(np.diff(b), -1.2 * np.diff(np.log(r)), atol=1e-5)


def test_mxfp4_config_quantises_the_prefill_weights():
    s = mi.Shape(T=4, H=64, E=3, k=2, I=32, mxfp4=True)
    a = mi.make(s, seed=1)
    b = mi.make(mi.Shape(T=4, H=64, E=3, k=2, I=32), seed=1)
    assert a.w_gate_up.shape == (3, 64, 32) and a.gu_scales.shape == (3, 64, 2)
    assert a.w_down.shape == (3, 64, 16) and a.d_scales.shape == (3, 64, 1)
    p, sc = mi.mxfp4_quantize(b.w_gate_up[1])
    assert (p == a.w_gate_up[1]).all() and (sc == a.gu_scales[1]).all()
    assert (a.x == b.x).all()
