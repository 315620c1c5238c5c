"""Host-side arithmetic of bench.py, on the CPU: the algorithmic bytes and
FLOPs the roofline figures divide by, the choice of the binding roofline, the
guard that drops stored HBM traffic counters once the kernel source changes,
and the one-GPU rule of the command line.

The expected figures are closed forms of the layer's shape (bf16 = 2 bytes;
MXFP4 = half a byte per value plus an E8M0 byte per 32; NVFP4 = half a byte
per value plus an E4M3 byte per 16 plus one fp32 matrix scale), written out
here independently of bench.algorithmic."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402

H, E, K, I = 2816, 128, 8, 704


def _alg(T, U, **fmt):
    s = mi.Shape(T=T, H=H, E=E, k=K, I=I, **fmt)
    ids = np.arange(U, dtype=np.int32)          # U distinct experts touched
    return bench.algorithmic(SimpleNamespace(shape=s), ids)


def test_per_expert_weight_bytes():
    assert _alg(8, 45)["gu_bytes_per_expert"] == 2 * 704 * 2816 * 2 == 7_929_856
    assert _alg(8, 45, mxfp4=True)["gu_bytes_per_expert"] == 1408 * (1408 + 88) == 2_106_368
    assert _alg(8, 45, nvfp4=True)["gu_bytes_per_expert"] == 1408 * (1408 + 176) + 4 == 2_230_276


def test_decode_bytes_and_flops():
    a = _alg(8, 45)
    # gate/up kernel: the 45 touched experts' [1408][2816] bf16 slabs, x (8 rows), h (64 rows of 704)
    assert a["gateup_bytes"] == 45 * 7_929_856 + 8 * 2816 * 2 + 64 * 704 * 2 == 356_978_688
    assert a["gateup_flops"] == 64 * 2 * 2816 * 1408
    # layer: touched experts' gate/up and down weights, the router weight, x in and out
    assert a["layer_bytes"] == 45 * (7_929_856 + 2816 * 704 * 2) + 128 * 2816 * 2 + 2 * 8 * 2816 * 2
    # per token: router 2HE, and k experts of 2*H*2I (gate/up) + 2*I*H (down)
    assert a["layer_flops"] == 8 * 95_879_168


def test_prefill_layer_figures():
    a = _alg(2048, 128)
    assert a["layer_bytes"] == 1_546_321_920
    assert a["layer_flops"] == 196_360_536_064
    # 0.41 of the bf16 peak is all the prefill shape can reach at the full 8 TB/s
    t_hbm = a["layer_bytes"] / 8e12
    assert a["layer_flops"] / t_hbm / 2.5e15 == pytest.approx(0.4068, abs=1e-3)


def test_dense_mlp_adds_its_weights_once():
    base, mlp = _alg(8, 45), _alg(8, 45, I_sh=2112)
    assert mlp["layer_bytes"] - base["layer_bytes"] == 2 * 2112 * 2816 * 2 + 2816 * 2112 * 2
    assert mlp["layer_flops"] - base["layer_flops"] == 8 * (2 * 2816 * 2 * 2112 + 2 * 2112 * 2816)


def test_binding_roofline():
    # decode and prefill sit below the ridge (312.5 FLOP/B): HBM binds
    for T, U in ((8, 45), (2048, 128)):
        r = bench.kernel_roofline(_alg(T, U), 100.0, bench.BF16_PEAK_TFLOPS)
        assert r["bound"] == "hbm" and r["unit"] == "GB/s"
        assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    # the 8192-token batch is above it: the matrix cores bind
    r = bench.kernel_roofline(_alg(8192, 128), 600.0, bench.BF16_PEAK_TFLOPS)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(65536 * 2 * 2816 * 1408 / 600e-6 / 1e12)
    lay = bench.layer_roofline(_alg(2048, 128), 0.42, bench.BF16_PEAK_TFLOPS)
    assert lay["binding"] == "hbm" and lay["binding_frac"] == max(lay["hbm_frac"], lay["mfma_frac"])


def test_traffic_guard(tmp_path, monkeypatch):
    """Stored counters are reported only while the kernel source they were
    taken on is unchanged."""
    (tmp_path / "profiles").mkdir()
    rec = {"kernel_source_hash": "abc123", "hbm_bytes_per_launch": 12345.0}
    (tmp_path / "profiles" / "gateup_demo_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    assert bench.traffic_from_profiles("demo") == 12345.0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.traffic_from_profiles("demo") is None
    assert bench.traffic_from_profiles("absent") is None


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "mixture_experts_router_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "moe_common.h").write_text("int a;\n")
    (src / "grouped_gemm.hip").write_text("int b = 1; // note\n/* block */ int c;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (src / "grouped_gemm.hip").write_text("int b = 1;   // another note\n  int c;\n")
    assert bench.kernel_source_hash() == h0
    (src / "grouped_gemm.hip").write_text("int b = 2;\nint c;\n")
    assert bench.kernel_source_hash() != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
