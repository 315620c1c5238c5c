"""Benchmark of the MoE FFN layer (moe_forward) on one MI355X.

A step is one moe_forward call over one batch of synthetic tokens: router
GEMM + top-k softmax, permutation, grouped gate/up GEMM + GEGLU, grouped
down GEMM, weighted combine.  The default workload is the Gemma-4-26B-A4B MoE
layer at decode size (T=8 tokens, hidden 2816, 128 experts, top-8,
intermediate 704, bf16).  Inputs are resident in HBM before timing; expert
weights rotate over several device copies so the 256 MB Infinity Cache
cannot serve them from a previous step.

Prints one JSON line:  value = tokens/s of the whole layer; roofline = the
dominant kernel (grouped gate/up GEMM) against the HBM or MFMA peak, its
duration from HIP events around back-to-back launches on the launch stream;
layer = the whole step against both rooflines; extra = the same figures for
the prefill-size workloads (bf16 prefill of 2048 tokens, the Zipf-skewed
prefill of 8192 tokens, MXFP4 experts), timed in the same process;
cpu_baseline = the fp64 numpy oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % HBM roofline (decode) / % bf16 MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense fp4 (MXFP4) MFMA
STAGES = ["route", "permute", "gateup", "down", "combine"]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="decode",
                   help="tiny|decode|prefill|skew|mxfp4|decode_shared|w4a4|mxfp4_decode|nvfp4_decode|"
                        "nvfp4_a4_decode|nvfp4_a4")
    p.add_argument("--rotate", type=int, default=4, help="device copies of the weights cycled per step")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    p.add_argument("--extra", default="prefill,skew,mxfp4",
                   help="other workloads timed in the same run and reported under 'extra' (comma list, or none)")
    p.add_argument("--extra-steps", type=int, default=30)
    p.add_argument("--extra-warmup", type=int, default=5)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a device copy of MIB mebibytes (counter calibration, copy bandwidth) and exit")
    p.add_argument("--stream-probe", action="store_true",
                   help="only time the load-only streaming probes (libmoe_probe.so) and exit")
    p.add_argument("--vendor-gemm", action="store_true",
                   help="only time the vendor library's bf16 matmul on the layer's expert shapes (context) and exit")
    return p.parse_args()


def algorithmic(inp, ids):
    """Bytes and flops the method must move/do (touched experts' weights once,
    router weight, x and out) for the layer and for the gate/up kernel."""
    s = inp.shape
    T, H, E, k, I = s.T, s.H, s.E, s.k, s.I
    U = int(np.unique(ids).size)
    if s.mxfp4:
        gu_bytes = 2 * I * (H // 2 + H // 32)
        d_bytes = H * (I // 2 + I // 32)
    elif s.nvfp4:   # codes, an E4M3 byte per 16 values, the fp32 matrix scale
        gu_bytes = 2 * I * (H // 2 + H // 16) + 4
        d_bytes = H * (I // 2 + I // 16) + 4
    else:
        gu_bytes = 2 * I * H * 2
        d_bytes = H * I * 2
    A = T * k
    layer_bytes = U * (gu_bytes + d_bytes) + E * H * 2 + 2 * T * H * 2
    layer_flops = T * (2 * H * E + k * (2 * H * 2 * I + 2 * I * H))
    gateup_bytes = U * gu_bytes + T * H * 2 + A * I * 2
    gateup_flops = A * 2 * H * 2 * I
    if s.I_sh:   # the dense MLP: its weights once, its FLOPs on every token
        Is = s.I_sh
        sh_gu = 2 * Is * (H // 2 + H // 32) if s.mxfp4 else 2 * Is * H * 2
        sh_d = H * (Is // 2 + Is // 32) if s.mxfp4 else H * Is * 2
        layer_bytes += sh_gu + sh_d
        layer_flops += T * (2 * H * 2 * Is + 2 * Is * H)
        gateup_bytes += sh_gu + T * Is * 2
        gateup_flops += T * 2 * H * 2 * Is
    return dict(U=U, layer_bytes=layer_bytes, layer_flops=layer_flops, gateup_bytes=gateup_bytes,
                gateup_flops=gateup_flops, gu_bytes_per_expert=gu_bytes)


def kernel_source_hash():
    """Hash of the gate/up kernel's code (comments and whitespace removed,
    so a comment edit does not invalidate counters taken on the same code)."""
    import re
    h = hashlib.sha256()
    for f in ("grouped_gemm.hip", "moe_common.h"):
        src = open(os.path.join(ROOT, "mixture_experts_router_amd", "csrc", f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(config):
    """HBM bytes per gate/up launch from a committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"gateup_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def host_info():
    """Where the numbers were taken: CPU model, BLAS threads, torch and HIP
    versions, the GPU and its compute units."""
    import torch
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:                                            # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                                          # pragma: no cover
        blas = None
    props = torch.cuda.get_device_properties(0)
    return {"cpu_model": cpu, "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": blas,
            "torch": torch.__version__, "hip": torch.version.hip, "gpu": props.name,
            "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count}


# The pages' own figures, for context only: whole-model latencies and rates on
# other hardware, none of them for this layer alone (so vs_baseline is null).
PAGES_CONTEXT = {
    "note": "whole-model figures from the pages on other hardware; none measures this layer",
    "ascend_910b_x8_bs8_seq256_prefill_ms": 312.51,
    "ascend_910b_x8_bs8_decode_ms": {"eager": 98.47, "after_operator_fusion": 92.0},
    "llama_cpp_rtx4070_iq3s_generation_tokens_per_s": 48,
}


def cpu_baseline(inp, budget_s):
    """The oracle as it stands, on this host, on a bounded sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                                          # pragma: no cover
        threads = 1
    s = inp.shape
    if s.T <= 64:
        t0 = time.perf_counter()
        n = 0
        while True:
            oracle.forward(inp)
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        tokens = n * s.T
        sample = f"{n} full oracle.forward calls on the T={s.T} workload"
    else:
        rng = np.random.default_rng(0)
        t0 = time.perf_counter()
        tokens = 0
        while time.perf_counter() - t0 < budget_s:
            tok = rng.choice(s.T, size=16, replace=False)
            oracle.forward_tokens(inp, tok)
            tokens += 16
        el = time.perf_counter() - t0
        sample = f"{tokens} tokens of the T={s.T} workload through oracle.forward_tokens (16 per call)"
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "seconds": round(el, 2),
            "host_cpus": len(os.sched_getaffinity(0))}


def kernel_roofline(alg, launch_us, mfma_peak):
    """The gate/up kernel against both rooflines; `bound` is the one its
    arithmetic intensity (FLOP per algorithmic byte) puts it under."""
    t = launch_us * 1e-6
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    gbs = alg["gateup_bytes"] / t / 1e9
    tfs = alg["gateup_flops"] / t / 1e12
    if alg["gateup_flops"] / alg["gateup_bytes"] > ridge:
        bound, unit, peak, achieved = "mfma", "TFLOP/s", mfma_peak, tfs
    else:
        bound, unit, peak, achieved = "hbm", "GB/s", HBM_PEAK_GBS, gbs
    return {"kernel": "grouped_gemm gate/up + GEGLU", "bound": bound, "achieved": achieved, "peak": peak,
            "unit": unit, "frac": achieved / peak, "hbm_frac": gbs / HBM_PEAK_GBS,
            "mfma_frac": tfs / mfma_peak, "alg_bytes_per_launch": alg["gateup_bytes"],
            "alg_flops_per_launch": alg["gateup_flops"], "avg_launch_us": launch_us}


def layer_roofline(alg, ms, mfma_peak):
    """The whole layer (one step) against both rooflines: t_roof / t with
    t_roof = max(F / peak, B / bandwidth) is the binding fraction."""
    t = ms * 1e-3
    layer = {"touched_experts": alg["U"], "alg_bytes": alg["layer_bytes"], "alg_flops": alg["layer_flops"],
             "hbm_frac": alg["layer_bytes"] / t / (HBM_PEAK_GBS * 1e9),
             "mfma_frac": alg["layer_flops"] / t / (mfma_peak * 1e12)}
    layer["binding_frac"] = max(layer["hbm_frac"], layer["mfma_frac"])
    layer["binding"] = "hbm" if layer["hbm_frac"] >= layer["mfma_frac"] else "mfma"
    return layer


def workload_name(config, s):
    return (f"Gemma-4-26B-A4B MoE FFN layer, {config}: T={s.T} tokens, "
            f"hidden {s.H}, {s.E} experts, top-{s.k}, intermediate {s.I}, "
            f"GEGLU, {'MXFP4' if s.mxfp4 else ('NVFP4' if s.nvfp4 else 'bf16')} expert weights"
            f"{' and MXFP4 activations (W4A4)' if s.a4 else ''}"
            f"{' and NVFP4 activations (W4A4)' if s.nv_a4 else ''}"
            f"{', Zipf(1.2) router bias' if s.skew else ''}"
            f"{f', plus the dense GEGLU MLP (intermediate {s.I_sh}) as a shared expert' if s.I_sh else ''}")


def measure(config, K, warmup, rotate, full):
    """Time moe_forward on one workload.  Returns (result dict, inputs).
    `full` adds the per-step event spread and the HIP-graph replay."""
    import torch
    import moe_inputs as mi
    import mixture_experts_router_amd as moe
    from mixture_experts_router_amd import device as dev

    t_gen = time.perf_counter()
    inp = mi.make(config, seed=0)
    s = inp.shape
    sh = moe.shape(s.T, s.H, s.E, s.k, s.I, mxfp4=s.mxfp4, a4=s.a4, nvfp4=s.nvfp4, nv_a4=s.nv_a4)
    x = dev.to_device(inp.x)
    wr = dev.to_device(inp.w_router)
    bias = dev.to_device(inp.router_bias) if inp.router_bias is not None else None
    gu0 = dev.to_device(inp.w_gate_up)
    d0 = dev.to_device(inp.w_down)
    gus = dev.to_device(inp.gu_scales) if s.mxfp4 else None
    ds = dev.to_device(inp.d_scales) if s.mxfp4 else None
    if s.nvfp4:   # one buffer per matrix: the fp32 expert scales (+ input scale), then the E4M3 codes
        gus = dev.to_device(moe.nvfp4_scale_buffer(inp.gu_global, inp.gu_scales,
                                                   inp.gu_input_scale if s.nv_a4 else 1.0))
        ds = dev.to_device(moe.nvfp4_scale_buffer(inp.d_global, inp.d_scales,
                                                  inp.d_input_scale if s.nv_a4 else 1.0))
    copies = [(gu0, d0)] + [(gu0.clone(), d0.clone()) for _ in range(max(0, rotate - 1))]
    if s.I_sh:   # the dense MLP's weights rotate with the experts'
        sg0, sd0 = dev.to_device(inp.w_sh_gate_up), dev.to_device(inp.w_sh_down)
        sh_copies = [(sg0, sd0)] + [(sg0.clone(), sd0.clone()) for _ in range(len(copies) - 1)]
        sgs = dev.to_device(inp.sh_gu_scales) if s.mxfp4 else None
        sds = dev.to_device(inp.sh_d_scales) if s.mxfp4 else None
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    ws = dev.workspace(sh, I_sh=s.I_sh)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen
    print(f"# inputs ready in {gen_s:.1f}s: {config} {s}", file=sys.stderr, flush=True)

    def step(i, events=None):
        gu, d = copies[i % len(copies)]
        if s.I_sh:
            sg, sd = sh_copies[i % len(copies)]
            moe.forward_shared(sh, x, wr, bias, gu, gus, d, ds, s.I_sh, sg, sgs, sd, sds, out, ids, wts, ws,
                               stage_events=events)
        else:
            moe.forward(sh, x, wr, bias, gu, gus, d, ds, out, ids, wts, ws, stage_events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy()
    alg = algorithmic(inp, ids_np)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    # Timed region 1: K plain steps -> ms_per_step and value.
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K

    # Timed region 2: K more steps with the library recording HIP events on
    # its launch stream between the stages -> per-kernel durations.  (An event
    # between two kernels adds a gap of a few microseconds, which is why the
    # step time comes from region 1.)
    ev = dev.StageEvents(K)
    torch.cuda.synchronize()
    for i in range(K):
        step(i, ev.arrays[i])
    torch.cuda.synchronize()
    stage_ms = np.array([ev.stage_ms(i) for i in range(K)])      # [K, 5]
    ev.close()
    stage_avg_us = {n: float(v) * 1e3 for n, v in zip(STAGES, stage_ms.mean(axis=0))}
    print(f"# {config}: {K} steps: {ms * 1e3:.1f} us/step; stages (us) " +
          " ".join(f"{n}={v:.1f}" for n, v in stage_avg_us.items()), file=sys.stderr, flush=True)

    # Timed region 3: the dominant kernel alone, K back-to-back launches of
    # moe_grouped_gemm_gateup on this step's routing (the weight copies
    # rotate as in region 1) -> its average launch duration for the roofline.
    A = s.T * s.k
    i32 = dict(dtype=torch.int32, device="cuda")
    r_logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    r_ids = torch.empty((s.T, s.k), **i32)
    r_w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(s.E, **i32)
    offsets = torch.empty(s.E + 1, **i32)
    sorted_ids = torch.empty(A, **i32)
    inv = torch.empty(A, **i32)
    h = torch.empty((A, s.I), dtype=torch.bfloat16, device="cuda")
    rws = torch.empty(max(1, moe.route_workspace_bytes(sh)), dtype=torch.uint8, device="cuda")
    pws = torch.empty(max(1, moe.permute_workspace_bytes(sh)), dtype=torch.uint8, device="cuda")
    moe.route(sh, x, wr, bias, r_logits, r_ids, r_w, ws=rws)
    moe.permute(sh, r_ids, None, counts, offsets, sorted_ids, inv, None, pws)
    torch.cuda.synchronize()
    if not torch.equal(r_ids.cpu(), ids.cpu()):
        raise RuntimeError("moe_route and moe_forward disagree on the routing")
    if s.I_sh or s.a4 or s.nv_a4:
        # the dense-MLP tiles (and the W4A4 GEMMs) run inside moe_forward
        # only: take the gate/up stage's duration from the stage events
        # (includes the gap an event adds, and for W4A4 the quantisation of x)
        gateup_launch_us = stage_avg_us["gateup"]
        print(f"# gate/up stage (stage events): {gateup_launch_us:.1f} us", file=sys.stderr, flush=True)
    else:
        moe.gemm_gateup(sh, x, sorted_ids, offsets, copies[0][0], gus, h)
        torch.cuda.synchronize()
        start.record()
        for i in range(K):
            moe.gemm_gateup(sh, x, sorted_ids, offsets, copies[i % len(copies)][0], gus, h)
        end.record()
        torch.cuda.synchronize()
        gateup_launch_us = start.elapsed_time(end) / K * 1e3
        print(f"# {config}: gate/up kernel alone: {gateup_launch_us:.1f} us per launch", file=sys.stderr,
              flush=True)

    spread, graph_us = None, None
    if full:
        # Timed region 4: K steps, each bracketed by its own pair of events ->
        # the spread of the step time (each pair adds its own record latency).
        ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            ev_a[i].record()
            step(i)
            ev_b[i].record()
        torch.cuda.synchronize()
        per_step = np.array([a.elapsed_time(b) * 1e3 for a, b in zip(ev_a, ev_b)])
        spread = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
                  "p90": float(np.percentile(per_step, 90))}
        # Timed region 5: the same steps captured once as a HIP graph (one
        # moe_forward per weight copy) and replayed back to back.
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(len(copies)):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, K // len(copies))
        start.record()
        for _ in range(reps):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        graph_us = start.elapsed_time(end) * 1e3 / (reps * len(copies))
        del g
        print(f"# per-step events p10/p50/p90 {spread['p10']:.1f}/{spread['p50']:.1f}/{spread['p90']:.1f} us; "
              f"graph replay {round(graph_us, 1)} us per step", file=sys.stderr, flush=True)

    mfma_peak = FP4_PEAK_TFLOPS if s.a4 else BF16_PEAK_TFLOPS   # the expert matmuls' own dtype
    roof = kernel_roofline(alg, gateup_launch_us, mfma_peak)
    roof["traffic"] = traffic_from_profiles(config)
    res = {
        "ms_per_step": ms,
        "tokens_per_s": s.T / (ms * 1e-3),
        "steps": K,
        "warmup": warmup,
        "dtype": "mxfp4" if s.a4 else "bf16",
        "config": {"workload": workload_name(config, s),
                   "T": s.T, "H": s.H, "E": s.E, "k": s.k, "I": s.I,
                   "weights": (("mxfp4 weights and activations (W4A4)" if s.a4 else "mxfp4") if s.mxfp4
                               else (("nvfp4 weights and activations (W4A4)" if s.nv_a4 else "nvfp4")
                                     if s.nvfp4 else "bf16")),
                   "weight_copies": len(copies),
                   **({"I_shared": s.I_sh} if s.I_sh else {})},
        "roofline": roof,
        "layer": layer_roofline(alg, ms, mfma_peak),
        "step_us": {"mean_back_to_back": ms * 1e3, "per_step_events": spread, "graph_replay": graph_us},
        "stages_us": stage_avg_us,
    }
    del copies, ws, out, h, x
    if s.I_sh:
        del sh_copies
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, inp


def vendor_gemm():
    """The vendor library's bf16 matmul (torch.bmm / torch.matmul, hipBLASLt)
    on the layer's expert shapes, for context: 128 experts x R rows each
    (batched, contiguous operands, no gather, no GEGLU epilogue) for the
    gate/up (K 2816 -> 1408) and down (K 704 -> 2816) products, and the same
    totals as one dense matrix.  TFLOP/s from HIP events over 20 calls."""
    import torch
    out = {}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def time(f, flops):
        f()
        torch.cuda.synchronize()
        start.record()
        for _ in range(20):
            f()
        end.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(end) / 20 * 1e3
        return {"us": round(us, 1), "tflops": round(flops / (us * 1e-6) / 1e12, 1)}

    for R in (128, 512):
        for name, K, N in (("gateup", 2816, 1408), ("down", 704, 2816)):
            a = torch.randn(128, R, K, device="cuda", dtype=torch.bfloat16)
            w = torch.randn(128, K, N, device="cuda", dtype=torch.bfloat16)   # [E][K][N]: contiguous right operand
            out[f"bmm_{name}_128x{R}"] = time(lambda: torch.bmm(a, w), 2.0 * 128 * R * K * N)
            del a, w
    for name, K, N in (("gateup", 2816, 1408), ("down", 704, 2816)):
        a = torch.randn(16384, K, device="cuda", dtype=torch.bfloat16)
        w = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
        out[f"dense_{name}_16384"] = time(lambda: torch.matmul(a, w), 2.0 * 16384 * K * N)
        del a, w
    torch.cuda.empty_cache()
    return {"vendor_gemm": out}


def stream_probe(launches=20):
    """The load-only streaming probes of libmoe_probe.so: a plain stream and
    the byte streams of the decode GEMMs' launch shapes, with no arithmetic,
    and the LDS read rate (16 waves per CU, conflict-free 16-byte reads).
    Each probe reads its bytes from one of four regions of a device buffer in
    turn (each region at least as large as the 256 MB Infinity Cache, so no
    launch finds its bytes there); us per launch from HIP events around
    `launches` back-to-back launches on the launch stream."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "mixture_experts_router_amd", "libmoe_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    lib.moe_probe_name.restype = ctypes.c_char_p
    lib.moe_probe_name.argtypes = [ctypes.c_int]
    lib.moe_probe_bytes.restype = ctypes.c_size_t
    lib.moe_probe_bytes.argtypes = [ctypes.c_int]
    lib.moe_probe_footprint.restype = ctypes.c_size_t
    lib.moe_probe_footprint.argtypes = [ctypes.c_int]
    lib.moe_probe_launch.restype = ctypes.c_int
    lib.moe_probe_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p]
    kinds = range(lib.moe_probe_count())
    region = max(max(lib.moe_probe_footprint(k) for k in kinds), 256 << 20)
    region = (region + (1 << 20) - 1) >> 20 << 20
    buf = torch.ones(4 * region, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def launch(k, i):
        rc = lib.moe_probe_launch(k, buf.data_ptr() + (i % 4) * region, region, sink.data_ptr(),
                                  stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"moe_probe_launch({k}) returned {rc}")

    out = []
    for k in kinds:
        for i in range(4):
            launch(k, i)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(launches):
            launch(k, i)
        end.record(stream)
        torch.cuda.synchronize()
        us = start.elapsed_time(end) / launches * 1e3
        nbytes = lib.moe_probe_bytes(k)
        out.append({"probe": lib.moe_probe_name(k).decode(), "bytes": nbytes, "us": round(us, 2),
                    "tb_per_s": round(nbytes / (us * 1e-6) / 1e12, 3)})
        if lib.moe_probe_footprint(k) == 0:   # the LDS probe: bytes per clock and CU at 2.4 GHz
            out[-1]["bytes_per_clk_per_cu_at_2p4ghz"] = round(nbytes / (us * 1e-6) / 2.4e9 / 256, 1)
        print(json.dumps(out[-1]), flush=True)
    del buf, sink
    torch.cuda.empty_cache()
    return {"stream_probe": out, "launches": launches}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the layer holds all experts on one device and the "
              f"library has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        # a device-to-device copy of known size: the counters' bytes per
        # copied byte, and the bandwidth a plain copy reaches (read + write)
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(3):
            b.copy_(a)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / 3
        print(json.dumps({"copy_calibration_bytes": n, "launches": 4, "copy_ms": ms,
                          "copy_read_plus_write_gbs": 2 * n / (ms * 1e-3) / 1e9}))
        return
    if args.vendor_gemm:
        print(json.dumps(vendor_gemm()))
        return
    if args.stream_probe:
        print(json.dumps(stream_probe()))
        return

    main_res, inp = measure(args.config, args.steps, args.warmup, args.rotate, full=not args.no_graph)
    # The other workloads of the metric, timed in the same process with the
    # same protocol (fewer steps): the prefill half of the metric (bf16
    # prefill, Zipf-skewed prefill, MXFP4 experts).
    extra = {}
    names = [] if args.extra in ("", "none") else [n for n in args.extra.split(",") if n != args.config]
    for name in names:
        r, _ = measure(name, args.extra_steps, args.extra_warmup, args.rotate, full=False)
        extra[name] = {key: r[key] for key in ("ms_per_step", "tokens_per_s", "steps", "warmup", "dtype",
                                               "config", "layer", "roofline", "stages_us")}
    res = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["dtype"],
        "data": "synthetic",
        "config": main_res["config"],
        "roofline": main_res["roofline"],
        "layer": main_res["layer"],
        "step_us": main_res["step_us"],
        "stages_us": main_res["stages_us"],
        "extra": extra,
        "host": host_info(),
        "context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
