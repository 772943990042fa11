"""Benchmark of the routed MoE FFN forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-ceilings]   # default workload: dsv3_bf16
    python bench.py --copy-calibration   # a plain 1 GiB device copy, for counter scaling
    python bench.py --compare-vendor qwen3,dsv3   # this grouped GEMM beside the vendor's
                                                  # batched GEMM on equal-row expert shapes

A step is one moe_ffn_forward over one batch: router, permute, grouped gate_up GEMM with
the fused activation, grouped down GEMM and combine (and the shared expert when the
workload has one). Inputs are seeded synthetic tensors already resident in HBM. W untimed
steps, then K timed steps between two device synchronisations; rank 0 prints one JSON
line. For the roofline entry the dominant kernel (the grouped gate_up GEMM) is timed
launch by launch with HIP events on the stream it runs on, inside complete layers run
through the separate entry points.
"""
import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mixture_experts_ffn_moerouter_amd import binding as B  # noqa: E402
from mixture_experts_ffn_moerouter_amd import inputs as I  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, TFLOP/s
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte where the roofs meet
METRIC = "MoE FFN tokens/s on 1 MI355X; % bf16 MFMA peak (prefill), % HBM BW (decode)"


# HBM bytes of one launch of a workload's dominant GEMM, read by the FETCH_SIZE and
# WRITE_SIZE counters (rocprofv3 --pmc, one counter per run, over this script's own
# launches; FP8 workloads with --host-inputs) and scaled by what the same counters read for
# a plain copy of known size (--copy-calibration). A figure belongs to the kernel code it
# was measured on: gemm_src is the SHA-256 of that kernel's file and csrc/tile_map.h with
# their comments and blank lines removed (gemm_source_digest), and different code reports
# null.
TRAFFIC = {
    # FETCH_SIZE KiB x 1.99995 + WRITE_SIZE KiB x 1.0 per launch (a 1 GiB copy read
    # 524301.3 KiB of FETCH_SIZE and wrote 1048576 KiB of WRITE_SIZE); layer inputs made on
    # the host (--host-inputs), profiles/gemm_<workload>_counters.md.
    # routed gate_up: 8376167.2 + 131072.0 KiB
    "dsv3_bf16": {"kernel": "gemm.hip", "bytes": 17288173022,
                  "gemm_src": "03eac19500d1e52b478a194bde0c3de9c1c9c7a68b1c6da5293a6db0b16a6c5d"},
    # routed gate_up: 526729.7 + 49152.1 KiB
    "qwen3_bf16": {"kernel": "gemm.hip", "bytes": 1129046837,
                   "gemm_src": "03eac19500d1e52b478a194bde0c3de9c1c9c7a68b1c6da5293a6db0b16a6c5d"},
    # FP8 (FETCH_SIZE x 1.99995 from that file's calibration),
    # profiles/gemm_fp8_masked_dsv3_traffic.md: 3791612.6 + 264821.8 KiB
    "dsv3_fp8_gate_up": {"kernel": "gemm_fp8.hip", "bytes": 8036203622,
                         "gemm_src": "65476cfa041b9c3bcf1e42f6b5a4464206460bd97f362ac527e192f6c034934e"},
    # 1895355.4 + 484635.7 KiB
    "dsv3_fp8_down": {"kernel": "gemm_fp8.hip", "bytes": 4377856522,
                      "gemm_src": "65476cfa041b9c3bcf1e42f6b5a4464206460bd97f362ac527e192f6c034934e"},
    # decode: one whole layer call (router, permute, both indexed kernels, combine),
    # profiles/moe_ffn_decode_dsv3_bf16_traffic.md: 4010184.5 + 15080.7 KiB
    "decode_dsv3_bf16": {"kernel": ("indexed.hip", "combine.hip"), "bytes": 8228095172,
                         "gemm_src": "c827bb773a1a558a5b6f378761cb902fb7c9aeb254ff5f3738fd81839692bc73"},
}


def code_text(src: str) -> str:
    """C++ source without its comments, trailing blanks and empty lines (the sources have
    no string literal holding a comment marker)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*$", "", line).rstrip() for line in src.splitlines())
    return "\n".join(line for line in lines if line)


def gemm_source_digest(kernel="gemm.hip") -> str:
    """SHA-256 over the code of a kernel's source (or a tuple of sources) and the tile-map
    header (comments do not count: editing one leaves the recorded figures valid)."""
    h = hashlib.sha256()
    for name in ((kernel,) if isinstance(kernel, str) else tuple(kernel)) + ("tile_map.h",):
        with open(os.path.join(ROOT, "mixture_experts_ffn_moerouter_amd", "csrc", name)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def recorded_traffic(workload: str):
    rec = TRAFFIC.get(workload)
    if rec is None or rec["gemm_src"] != gemm_source_digest(rec.get("kernel", "gemm.hip")):
        return None
    return rec["bytes"]


def copy_calibration():
    """1 GiB bf16 device-to-device copy, five times: 1 GiB read and 1 GiB written each."""
    n = 1 << 29
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "copies": 5}),
          flush=True)


def oracle_threads() -> int:
    """Threads the C oracle runs on: the CPUs this process may use, capped by
    OMP_NUM_THREADS when that is set (a host's share of cores for one GPU)."""
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cpus = os.cpu_count() or 1
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return max(1, min(cpus, cap) if cap > 0 else cpus)


def host_description(cores: int = 0) -> dict:
    """The CPU threads the baseline actually ran on (`cores`: the C oracle's worker
    threads, or the numpy oracle's BLAS threads when not given), the CPUs this process
    may run on, and the CPU model."""
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cpus = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"cores": cores or _blas_threads(), "host_cpus": cpus, "cpu_model": model,
            "os_cpu_count": os.cpu_count()}


def measured_ceilings(reps: int = 5) -> dict:
    """The device's attainable streaming-read bandwidth, L2-resident read rate and dense
    bf16 MFMA rate, from the probes of libmoe_probes.so (include/moe_probes.h), timed with
    HIP events on the current stream: a 4 GiB read with non-temporal 16-byte loads; a 1 MiB
    region read 4096 times per wave by one eight-wave workgroup per CU, in both load forms;
    four independent v_mfma_f32_32x32x16_bf16 chains per wave at two waves per SIMD. Best of
    `reps`."""
    path = os.path.join(ROOT, "mixture_experts_ffn_moerouter_amd", "libmoe_probes.so")
    L = ctypes.CDLL(path)
    L.moe_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p]
    L.moe_probe_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    grid = cus * 2
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")

    def read():
        rc = L.moe_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, sh)
        assert rc == 0, rc

    t_read = min(time_launches(read, 1, stream) for _ in range(reps))
    # L2-resident reads (a 1 MiB region), one workgroup of eight waves per CU
    L.moe_probe_l2_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_void_p]
    region, rounds = 1 << 20, 256
    l2 = {}
    for name, to_lds in (("lds", 1), ("registers", 0)):
        def l2read():
            rc = L.moe_probe_l2_read(buf.data_ptr(), region, rounds, to_lds, sink.data_ptr(),
                                     cus, sh)
            assert rc == 0, rc
        t = min(time_launches(l2read, 1, stream) for _ in range(reps))
        l2[name] = cus * 512 * 16 * 16 * rounds / (t * 1e-3)
    del buf
    iters = 20000
    mgrid = cus * 2  # 2 workgroups of four waves per CU: two waves per SIMD
    fsink = torch.zeros(mgrid, dtype=torch.float32, device="cuda")

    def mfma():
        rc = L.moe_probe_mfma_bf16(iters, fsink.data_ptr(), mgrid, sh)
        assert rc == 0, rc

    t_mfma = min(time_launches(mfma, 1, stream) for _ in range(reps))
    flops = mgrid * 4 * iters * 4 * 2 * 32 * 32 * 16
    return {"hbm_read_GBs": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops / (t_mfma * 1e-3) / 1e12, 1),
            "l2_read_to_lds_GBs": round(l2["lds"] / 1e9, 1),
            "l2_read_to_registers_GBs": round(l2["registers"] / 1e9, 1),
            "source": "probes/ceilings.hip (4 GiB non-temporal streaming read; 1 MiB "
                      "L2-resident region read by one 8-wave workgroup per CU, 16-byte loads "
                      "direct to LDS or into registers; bf16 32x32x16 MFMA loop)"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def distinct_experts(topk_ids: torch.Tensor) -> int:
    return int(torch.unique(topk_ids).numel())


def gate_up_algorithmic_bytes(cfg, n_experts: int) -> int:
    """Bytes the gate_up kernel must move at minimum: each touched expert's [2F, H] weights
    once, each token's hidden row once, each route's [F] activation row written once, and
    the route index / offsets metadata."""
    s = 4 if cfg.dtype == "f32" else 2
    R = cfg.T * cfg.K
    b = n_experts * 2 * cfg.F * cfg.H * s + cfg.T * cfg.H * s + R * cfg.F * s
    if cfg.bias_std is not None:
        b += n_experts * 2 * cfg.F * s
    return b + R * 4 + (cfg.E + 1) * 4


def gate_up_flops(cfg) -> int:
    return 2 * cfg.T * cfg.K * cfg.H * 2 * cfg.F


def layer_algorithmic(cfg, n_experts: int):
    """Whole-layer minimum bytes and flops (weights of touched experts read once, inputs
    read once, outputs written once, the activation written and read once)."""
    s = 4 if cfg.dtype == "f32" else 2
    R = cfg.T * cfg.K
    by = n_experts * 3 * cfg.F * cfg.H * s + cfg.T * cfg.H * s + cfg.T * cfg.E * 4 \
        + cfg.T * cfg.H * s + 2 * R * cfg.F * s
    fl = 6 * R * cfg.H * cfg.F
    if cfg.F_s:
        by += 3 * cfg.F_s * cfg.H * s + cfg.T * cfg.H * s + 2 * cfg.T * cfg.F_s * s
        fl += 6 * cfg.T * cfg.H * cfg.F_s
    return by, fl


def host_layer_inputs(cfg):
    """Counter runs of a layer workload: logits, bias, hidden and the shared expert are
    generated on the host (the same values as on the device), and expert 0's weights,
    generated on the host, are copied to every expert. The profiled process then launches
    no generator kernels; the routing, and so every kernel's byte traffic, is the
    workload's own (the GEMMs' traffic does not depend on the weight values)."""
    d = {k: v.to("cuda") for k, v in I.make_router_inputs(cfg, device="cpu").items()}
    dt = cfg.torch_dtype
    d["hidden"] = I.normal((cfg.T, cfg.H), cfg.x_std, seed=0, stream=I.STREAMS["hidden"],
                           dtype=dt).to("cuda")
    for name, shape in (("w_gate_up", (2 * cfg.F, cfg.H)), ("w_down", (cfg.H, cfg.F))):
        one = I.normal((1,) + shape, cfg.w_std, seed=0, stream=I.STREAMS[name], dtype=dt)
        d[name] = one.to("cuda").expand(cfg.E, *shape).contiguous()
    if cfg.bias_std is not None:
        for name, n in (("b_gate_up", 2 * cfg.F), ("b_down", cfg.H)):
            d[name] = I.normal((cfg.E, n), cfg.bias_std, seed=0, stream=I.STREAMS[name],
                               dtype=dt).to("cuda")
    if cfg.F_s:
        d["shared_w_gate_up"] = I.normal((2 * cfg.F_s, cfg.H), cfg.w_std, seed=0,
                                         stream=I.STREAMS["shared_w_gate_up"],
                                         dtype=dt).to("cuda")
        d["shared_w_down"] = I.normal((cfg.H, cfg.F_s), cfg.w_std, seed=0,
                                      stream=I.STREAMS["shared_w_down"], dtype=dt).to("cuda")
    return d


def run_layer(cfg, d, fcfg, ws, out, shared_out):
    B.moe_ffn_forward(fcfg, d["hidden"], d["logits"], d["w_gate_up"], d["w_down"],
                      d.get("correction_bias"), d.get("expert_ids"), d.get("b_gate_up"),
                      d.get("b_down"), d.get("shared_w_gate_up"), d.get("shared_w_down"),
                      out=out, shared_out=shared_out, workspace=ws)


def time_launches(call, reps: int, stream) -> float:
    """Average duration in ms of one call, HIP events recorded around each launch on the
    stream the kernels run on."""
    for _ in range(3):
        call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


# Equal-row per-expert shapes (experts, rows per expert, K, N) on which this library's
# grouped GEMM and the vendor library's batched GEMM (torch.bmm) can run the same product:
# no gather, no activation, the same operands. gate_up: K = H, N = 2F; down: K = F, N = H.
VENDOR_SHAPES = {"qwen3": (128, 256, 2048, 1536), "dsv3": (256, 128, 7168, 4096),
                 "qwen3_down": (128, 256, 768, 2048), "dsv3_down": (256, 128, 2048, 7168)}


def compare_vendor(names, reps: int):
    """moe_grouped_gemm and torch.bmm (hipBLASLt on this image) on the same equal-row expert
    shapes: a [E*m, K] token rows, b [E, N, K] weights; the vendor call takes b as a
    contiguous [E, K, N] copy (its right operand must not be a transposed view). HIP events
    around each launch; one JSON line per shape (a measurement aid, not the bench line)."""
    s = torch.cuda.current_stream()
    for name in names:
        E, m, K, N = VENDOR_SHAPES[name]
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn((E * m, K), device="cuda", generator=g).to(torch.bfloat16)
        b = (0.02 * torch.randn((E, N, K), device="cuda", generator=g)).to(torch.bfloat16)
        bt = b.transpose(1, 2).contiguous()
        off = torch.arange(0, E * m + 1, m, dtype=torch.int32, device="cuda")
        out = torch.empty((E * m, N), dtype=torch.bfloat16, device="cuda")
        out_v = torch.empty((E, m, N), dtype=torch.bfloat16, device="cuda")
        ours = lambda: B.moe_grouped_gemm(a, b, off, None, out=out, stream=s)
        vendor = lambda: torch.bmm(a.view(E, m, K), bt, out=out_v)
        t_ours, t_vendor = time_launches(ours, reps, s), time_launches(vendor, reps, s)
        diff = float((out.view(E, m, N).float() - out_v.float()).abs().max())
        nbytes = E * N * K * 2 + E * m * K * 2 + E * m * N * 2
        print(json.dumps({"compare": "grouped GEMM vs vendor batched GEMM", "shape": name,
                          "experts": E, "rows_per_expert": m, "K": K, "N": N,
                          "ours_ms": round(t_ours, 4), "vendor_ms": round(t_vendor, 4),
                          "bytes": nbytes, "max_abs_diff": diff}), flush=True)


def time_burst(call, reps: int, stream) -> float:
    """Average duration in ms of one call over back-to-back launches, HIP events around the
    whole burst on the stream the kernels run on (for calls shorter than their host-side
    launch cost, where events around each launch would time the host)."""
    for _ in range(3):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_gate_up(cfg, d, reps: int):
    """Average duration of the grouped gate_up GEMM launch, timed inside complete layers.

    Each repetition runs the staged layer through the boundary's separate entry points
    (route, permute, gate_up, down, combine: the kernels moe_ffn_forward launches) and
    brackets only the gate_up launch with HIP events on its stream. Timing the kernel in a
    loop of its own would measure it at the lower clock that back-to-back heavy GEMMs drive
    the chip to, not at the one it runs at in the layer."""
    stream = torch.cuda.current_stream()
    rcfg = B.route_cfg(cfg.K, cfg.scoring, cfg.renormalize, cfg.rsf, cfg.G, cfg.TG)
    act = torch.empty((cfg.T * cfg.K, cfg.F), dtype=cfg.torch_dtype, device="cuda")
    y = torch.empty((cfg.T * cfg.K, cfg.H), dtype=cfg.torch_dtype, device="cuda")
    out = torch.empty((cfg.T, cfg.H), dtype=cfg.torch_dtype, device="cuda")
    ids = None

    def layer(a=None, b=None):
        nonlocal ids
        w, ids, _, _ = B.moe_route(d["logits"], rcfg, d.get("correction_bias"),
                                   d.get("expert_ids"), stream=stream)
        off, srt, pos, _ = B.moe_permute(ids, cfg.E, stream=stream)
        if a is not None:
            a.record(stream)
        B.moe_grouped_gemm_swiglu(d["hidden"], d["w_gate_up"], off, cfg.act,
                                  d.get("b_gate_up"), a_rows=srt, a_rows_div=cfg.K, out=act,
                                  stream=stream)
        if b is not None:
            b.record(stream)
        B.moe_grouped_gemm(act, d["w_down"], off, d.get("b_down"), out=y, stream=stream)
        B.moe_combine(y, w, pos, out=out, stream=stream)

    for _ in range(3):
        layer()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        layer(a, b)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(ms)), distinct_experts(ids)


def router_line(cfg, args):
    """Router-only workload: moe_route with the expert-parallel outputs, launch-bound.

    value = tokens per second of one routing call; roofline against HBM over the bytes the
    call must move (logits and bias in, ids, weights, router_probs and weight_scale out)."""
    d = I.make_router_inputs(cfg, device="cuda")
    rcfg = B.route_cfg(cfg.K, cfg.scoring, cfg.renormalize, cfg.rsf, cfg.G, cfg.TG,
                       cfg.local_expert_start, cfg.local_expert_count or 0,
                       cfg.router_probs_dtype or "f32")
    stream = torch.cuda.current_stream()
    ep = cfg.local_expert_count is not None
    # One routing call is a few microseconds of GPU work, less than the Python binding
    # spends marshalling a call. The timed calls therefore go to the C ABI the way a
    # native caller makes them: outputs allocated and arguments marshalled once.
    w, ids, rp, ws = B.moe_route(d["logits"], rcfg, d.get("correction_bias"),
                                 d.get("expert_ids"), with_router_probs=ep, stream=stream)
    c = B.MoeRouteCfg.from_buffer_copy(rcfg)
    c.logits_dtype = B.TORCH_DTYPES[d["logits"].dtype]
    raw = (B._ptr(d["logits"]), cfg.T, cfg.E, B._ptr(d.get("correction_bias")),
           B._ptr(d.get("expert_ids")), ctypes.byref(c), B._ptr(w), B._ptr(ids), B._ptr(rp),
           B._ptr(ws), B._stream(stream))
    lib = B.lib()
    B._check("moe_route", lib.moe_route(*raw))
    call = lambda: lib.moe_route(*raw)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    k_ms = time_burst(call, args.kernel_reps, stream)
    rp = 2 if cfg.router_probs_dtype in ("f16", "bf16") else 4
    lg = 2 if cfg.logits_dtype in ("f16", "bf16") else 4
    k_bytes = cfg.T * cfg.E * lg + (cfg.E * 4 if cfg.correction_bias else 0) \
        + cfg.T * cfg.K * 8 + ((cfg.local_expert_count + 1) * cfg.T * rp if ep else 0)
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(cfg.T / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded SplitMix64/Box-Muller logits)",
        "config": {"workload": cfg.name, "T": cfg.T, "E": cfg.E, "top_k": cfg.K,
                   "scoring": cfg.scoring, "logits_dtype": cfg.logits_dtype,
                   "num_expert_group": cfg.G, "topk_group": cfg.TG,
                   "local_expert_start": cfg.local_expert_start,
                   "local_expert_count": cfg.local_expert_count,
                   "router_probs_dtype": cfg.router_probs_dtype, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 6),
                     "traffic": None,
                     "kernel": "router kernel of moe_route" + (" (launch-bound: tiny input)"
                                                                 if cfg.T <= 64 else ""),
                     "kernel_ms": round(k_ms, 5), "latency_us": round(k_ms * 1e3, 2),
                     "algorithmic_bytes": k_bytes},
    }
    if not args.no_cpu_baseline:
        from oracle.c_oracle import load
        Cx = load(1)  # the C router takes one row after another on one thread
        logits = d["logits"].cpu()
        bias = None if d.get("correction_bias") is None else \
            d["correction_bias"].cpu().numpy().astype(np.float64)
        rp = cfg.router_probs_dtype if cfg.local_expert_count else None
        done, total = 0, 0.0
        n = min(cfg.T, 256)
        while total < args.cpu_budget / 4:
            t1 = time.perf_counter()
            Cx.route(logits[:n], cfg.K, cfg.scoring, cfg.renormalize, cfg.rsf, cfg.G, cfg.TG,
                     bias, None, cfg.local_expert_start, cfg.local_expert_count or None, rp)
            total += time.perf_counter() - t1
            done += n
        line["cpu_baseline"] = {"value": done / total, "unit": "tokens/s",
                                **host_description(1), "kind": "oracle",
                                "sample": f"first {n} of {cfg.T} tokens, repeated "
                                          f"({done} routed), float64 C oracle "
                                          f"(oracle/moe_ref.c), one thread, {total:.1f} s"}
    print(json.dumps(line), flush=True)


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def swiglu_line(cfg, args):
    """Standalone SwiGLU operator: one call per step over [rows, 2F] -> [rows, F]; value =
    rows per second; roofline against HBM over the bytes the op must move."""
    d = I.make_swiglu_inputs(cfg, device="cuda")
    out = torch.empty((cfg.rows, cfg.F), dtype=d["gate"].dtype, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: B.moe_swiglu(d["gate"], None, cfg.alpha, cfg.beta, cfg.limit, cfg.fusion,
                                out=out, stream=stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    k_ms = time_burst(call, args.kernel_reps, stream)
    es = 4 if cfg.dtype == "f32" else 2
    k_bytes = cfg.rows * cfg.F * 3 * es
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(cfg.rows / (ms_per_step * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype + " storage, f32 arithmetic",
        "data": "synthetic (seeded SplitMix64/Box-Muller values)",
        "config": {"workload": cfg.name, "rows": cfg.rows, "F": cfg.F, "fusion": cfg.fusion,
                   "alpha": cfg.alpha, "beta": cfg.beta, "limit": cfg.limit,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "swiglu_vec_kernel (standalone SwiGLU)",
                     "kernel_ms": round(k_ms, 5), "algorithmic_bytes": k_bytes},
    }
    if not args.no_cpu_baseline:
        from oracle.c_oracle import load
        Cx = load(1)  # the C activation runs element after element on one thread
        x = d["gate"][:512].float().cpu().numpy().astype(np.float64)
        done, total = 0, 0.0
        while total < args.cpu_budget / 4:
            t1 = time.perf_counter()
            Cx.swiglu_op(x, None, cfg.alpha, cfg.beta, cfg.limit, cfg.fusion, cfg.dtype)
            total += time.perf_counter() - t1
            done += x.shape[0]
        line["cpu_baseline"] = {"value": done / total, "unit": "rows/s",
                                **host_description(1), "kind": "oracle",
                                "sample": f"first 512 of {cfg.rows} rows, repeated ({done} "
                                          f"rows), float64 C oracle (oracle/moe_ref.c), one "
                                          f"thread, {total:.1f} s"}
    print(json.dumps(line), flush=True)


def _timed_line(call, args, stream, burst: bool = False):
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    timer = time_burst if burst else time_launches
    return ms_per_step, timer(call, args.kernel_reps, stream)


def layout_line(cfg, args):
    """Layout workloads: moe_pre_permute of a workload's routing into block-aligned rows
    (value = routes per second), or the bf16 grouped GEMM over a masked slab (value =
    valid rows / 8 per second, as the FP8 lines). Roofline against HBM."""
    stream = torch.cuda.current_stream()
    import oracle.moe_oracle as O
    if cfg.kind == "pre_permute":
        mc = I.CONFIGS[cfg.route]
        d = I.make_inputs(mc, device="cuda")
        _, ids, _, _ = B.moe_route(d["logits"], B.route_cfg(mc.K, mc.scoring, mc.renormalize,
                                                            mc.rsf, mc.G, mc.TG))
        ws = torch.empty(B.moe_layout_workspace_size(mc.T, mc.K, mc.E, cfg.block_size),
                         dtype=torch.uint8, device="cuda")
        call = lambda: B.moe_pre_permute(d["hidden"], ids, mc.E, cfg.layout, cfg.block_size,
                                         workspace=ws, stream=stream)
        ms, k_ms = _timed_line(call, args, stream, burst=True)
        R = mc.T * mc.K
        es = 4 if mc.dtype == "f32" else 2
        k_bytes = mc.T * mc.H * es + R * mc.H * es + R * 4 + R * 4 + mc.E * 4
        value, unit = R / (ms * 1e-3), "routes/s"
        conf = {"workload": cfg.name, "T": mc.T, "top_k": mc.K, "E": mc.E, "H": mc.H,
                "layout": cfg.layout, "block_size": cfg.block_size}
        kernel = "permute + align_rows_kernel (the whole op)"
        dtype = mc.dtype
        sample = None
        if not args.no_cpu_baseline:
            h = d["hidden"][:512].float().cpu().numpy().astype(np.float64)
            ii = ids[:512].cpu().numpy()
            done, total = 0, 0.0
            while total < args.cpu_budget / 4:
                t1 = time.perf_counter()
                O.pre_permute(h, ii, mc.E, cfg.layout, cfg.block_size)
                total += time.perf_counter() - t1
                done += ii.size
            sample = {"value": done / total, "unit": "routes/s", **host_description(),
                      "kind": "oracle", "sample": f"first 512 of {mc.T} tokens ({ii.size} "
                      f"routes), repeated, float64 numpy oracle, {total:.1f} s"}
    else:
        fc = I.FP8_CONFIGS[cfg.fp8]
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn((fc.E, fc.max_m, fc.K), device="cuda", generator=g).to(torch.bfloat16)
        w = (cfg.w_std * torch.randn((fc.E, fc.N, fc.K), device="cuda", generator=g)).to(
            torch.bfloat16)
        counts = I.fp8_counts(fc, device="cuda")
        out = torch.empty((fc.E, fc.max_m, fc.N), dtype=torch.bfloat16, device="cuda")
        call = lambda: B.moe_grouped_gemm_layout(a, w, "masked", counts, out=out, stream=stream)
        ms, k_ms = _timed_line(call, args, stream)
        rows = int(counts.cpu().clamp(0, fc.max_m).sum())
        k_bytes = fc.E * fc.N * fc.K * 2 + rows * fc.K * 2 + rows * fc.N * 2 + fc.E * 4
        value, unit = rows / 8 / (ms * 1e-3), "tokens/s"
        conf = {"workload": cfg.name, "E": fc.E, "max_m": fc.max_m, "K": fc.K, "N": fc.N,
                "valid_rows": rows, "layout": "masked"}
        kernel = "gemm_h16_kernel (grouped GEMM, masked slab)"
        dtype = "bf16"
        sample = None
        if not args.no_cpu_baseline:
            cnt = counts.cpu().numpy()
            done, total, e = 0, 0.0, 0
            while total < args.cpu_budget / 2 and e < fc.E:
                ae, we = a[e:e + 1].float().cpu().numpy(), w[e:e + 1].float().cpu().numpy()
                t1 = time.perf_counter()
                O.grouped_gemm_layout(ae, we, "masked", cnt[e:e + 1], None, None, "bf16")
                total += time.perf_counter() - t1
                done += int(cnt[e])
                e += 1
            sample = {"value": done / 8 / total, "unit": "tokens/s", **host_description(),
                      "kind": "oracle", "sample": f"experts 0..{e - 1} of {fc.E} ({done} valid "
                      f"rows), float64 numpy oracle, {total:.1f} s"}
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded inputs)", "config": {**conf, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": kernel, "kernel_ms": round(k_ms, 5), "algorithmic_bytes": k_bytes},
    }
    if sample:
        line["cpu_baseline"] = sample
    print(json.dumps(line), flush=True)


def fp8_line(cfg, args):
    """Block-scaled FP8 grouped GEMM over a masked slab (one step = one call). tokens =
    valid rows / 8 (the workload is the top-8 routed GEMM of T tokens)."""
    if args.host_inputs:
        # Counter runs: expert 0 is generated on the host and copied to every expert, so
        # the profiled process launches no generator kernels (the byte traffic of the GEMM
        # does not depend on the values).
        one = I.make_fp8_inputs(dataclasses.replace(cfg, E=1, counts=(0,)), device="cpu")
        d = {k: one[k].expand(cfg.E, *one[k].shape[1:]).contiguous().to("cuda")
             for k in ("a", "a_scale", "b", "b_scale")}
        d["counts"] = I.fp8_counts(cfg, device="cpu").to("cuda")
    else:
        d = I.make_fp8_inputs(cfg, device="cuda")
    out = torch.empty((cfg.E, cfg.max_m, cfg.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: B.moe_grouped_gemm_fp8_masked(d["a"], d["a_scale"], d["b"], d["b_scale"],
                                                 d["counts"], out=out, stream=stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    k_ms = time_launches(call, args.kernel_reps, stream)
    counts = d["counts"].cpu().numpy().astype(np.int64)
    rows = int(counts.sum())
    tokens = rows / 8.0
    nkb = cfg.K // 128
    k_bytes = rows * cfg.K + cfg.E * cfg.N * cfg.K + rows * nkb * 4 \
        + cfg.E * (cfg.N // 128) * nkb * 4 + cfg.E * 4 + rows * cfg.N * 2
    k_flops = 2 * rows * cfg.N * cfg.K
    if k_flops / k_bytes > FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(k_flops / (k_ms * 1e-3) / 1e12, 1),
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(k_bytes / (k_ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    line = {
        "metric": METRIC, "value": round(tokens / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 e4m3fn (block-scaled), fp32 accumulate, bf16 out",
        "data": "synthetic (seeded SplitMix64/Box-Muller values, block-quantized to e4m3fn)",
        "config": {"workload": cfg.name, "E": cfg.E, "max_m": cfg.max_m, "K": cfg.K,
                   "N": cfg.N, "valid_rows": rows, "parallelism": "single GPU"},
        "roofline": {**roof, "traffic": recorded_traffic(cfg.name),
                     "kernel": "gemm_fp8_masked_kernel (block-scaled FP8 grouped GEMM)",
                     "kernel_ms": round(k_ms, 4), "algorithmic_bytes": k_bytes,
                     "algorithmic_flops": k_flops},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        from oracle.c_oracle import load
        threads = oracle_threads()
        Cx = load(threads)
        done, total, g = 0, 0.0, 0
        while total < args.cpu_budget / 2 and g < cfg.E:
            sub = {k: v[g:g + 1].cpu().numpy() for k, v in d.items() if k != "counts"}
            t1 = time.perf_counter()
            Cx.grouped_gemm_fp8_masked(sub["a"].view(np.uint8), sub["a_scale"],
                                       sub["b"].view(np.uint8), sub["b_scale"], counts[g:g + 1])
            total += time.perf_counter() - t1
            done += int(counts[g])
            g += 1
        line["cpu_baseline"] = {
            "value": done / 8.0 / total, "unit": "tokens/s", **host_description(threads),
            "kind": "oracle",
            "sample": f"experts 0..{g - 1} of {cfg.E} ({done} of {rows} valid rows), float64 "
                      f"C oracle (oracle/moe_ref.c) on {threads} threads, {total:.1f} s"}
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, d, budget_s: float):
    """The C oracle (oracle/moe_ref.c), as it stands, on the first n tokens of the same
    workload: inputs in their storage formats on the host, one token per worker thread at
    a time, on every CPU this process may use."""
    from oracle.c_oracle import load
    threads = oracle_threads()
    Cx = load(threads)
    host = {k: v.cpu() for k, v in d.items()}
    bias = host.get("correction_bias")
    kw = dict(top_k=cfg.K, scoring=cfg.scoring, renormalize=cfg.renormalize,
              routed_scaling_factor=cfg.rsf, num_expert_group=cfg.G, topk_group=cfg.TG,
              act=cfg.act, dtype=cfg.dtype,
              correction_bias=None if bias is None else bias.double().numpy(),
              b_gate_up=host.get("b_gate_up"), b_down=host.get("b_down"),
              shared_w_gate_up=host.get("shared_w_gate_up"),
              shared_w_down=host.get("shared_w_down"))
    ids = host.get("expert_ids")

    def run(n):
        t0 = time.perf_counter()
        Cx.moe_ffn_forward(host["hidden"][:n], host["logits"][:n], host["w_gate_up"],
                           host["w_down"], expert_ids=None if ids is None else ids[:n], **kw)
        return time.perf_counter() - t0
    n = min(cfg.T, threads)
    while True:  # grow the sample until one pass takes a third of the budget
        dt = run(n)
        if dt >= budget_s / 3 or n >= cfg.T:
            break
        n = min(cfg.T, n * 4)
    passes, total = 1, dt
    while total < budget_s / 2:  # whole workload is quick: repeat it to about 10 s
        total += run(n)
        passes += 1
    res = {"value": n * passes / total, "unit": "tokens/s", **host_description(threads),
           "kind": "oracle",
           "sample": f"first {n} of {cfg.T} tokens of the same workload, {passes} pass(es), "
                     f"float64 C oracle (oracle/moe_ref.c) on {threads} threads, "
                     f"{total:.1f} s wall"}
    if cfg.T <= 64 and threads > 1:
        # small batches (the tiny and decode layers): the whole batch on one thread too
        C1, t0 = load(1), time.perf_counter()
        C1.moe_ffn_forward(host["hidden"], host["logits"], host["w_gate_up"], host["w_down"],
                           expert_ids=ids, **kw)
        wall = time.perf_counter() - t0
        res["single_thread"] = {"value": cfg.T / wall, "unit": "tokens/s",
                                "wall_s": round(wall, 3), "sample": f"all {cfg.T} tokens"}
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_bf16",
                    choices=sorted(I.CONFIGS) + sorted(I.FP8_CONFIGS) + sorted(I.SWIGLU_CONFIGS)
                    + sorted(I.LAYOUT_CONFIGS))
    ap.add_argument("--backend", default="auto", choices=["auto", "staged", "indexed"])
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--compare-vendor", default=None,
                    help="comma list of " + ",".join(VENDOR_SHAPES) + ": this grouped GEMM "
                         "and torch.bmm on the same equal-row expert shapes")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured stream-read and MFMA-loop ceilings")
    ap.add_argument("--host-inputs", action="store_true",
                    help="FP8 and layer workloads: host-generated inputs, one expert's weights "
                         "copied to every expert (counter runs; the traffic is unchanged)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the path is built and measured on a single "
              "MI355X (no collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.compare_vendor:
        compare_vendor(args.compare_vendor.split(","), args.kernel_reps)
        return
    if args.workload in I.FP8_CONFIGS:
        torch.cuda.set_device(0)
        fp8_line(I.FP8_CONFIGS[args.workload], args)
        return
    if args.workload in I.SWIGLU_CONFIGS:
        torch.cuda.set_device(0)
        swiglu_line(I.SWIGLU_CONFIGS[args.workload], args)
        return
    if args.workload in I.LAYOUT_CONFIGS:
        torch.cuda.set_device(0)
        layout_line(I.LAYOUT_CONFIGS[args.workload], args)
        return
    cfg = I.CONFIGS[args.workload]
    if cfg.H == 0:
        torch.cuda.set_device(0)
        router_line(cfg, args)
        return
    torch.cuda.set_device(0)
    log(f"[bench] {cfg.name}: generating inputs" + (" on the host" if args.host_inputs else ""))
    d = host_layer_inputs(cfg) if args.host_inputs else I.make_inputs(cfg, device="cuda")
    fcfg = B.ffn_cfg(cfg, args.backend)
    backend = {1: "staged", 2: "indexed"}[B.moe_ffn_backend(fcfg, cfg.bias_std is not None)]
    ws = torch.empty(B.moe_ffn_workspace_size(fcfg), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.H), dtype=cfg.torch_dtype, device="cuda")
    shared_out = torch.empty_like(out) if cfg.F_s else None
    log(f"[bench] backend {backend}; warmup {args.warmup}")
    for _ in range(args.warmup):
        run_layer(cfg, d, fcfg, ws, out, shared_out)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_layer(cfg, d, fcfg, ws, out, shared_out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    tokens_per_s = cfg.T * args.steps / elapsed
    # the spread of single steps, from HIP events around each layer in a second pass (the
    # timed region above has no events in it)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        run_layer(cfg, d, fcfg, ws, out, shared_out)
        b.record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in evs]

    _, ids, _, _ = B.moe_route(d["logits"], B.route_cfg(cfg.K, cfg.scoring, cfg.renormalize,
                                                        cfg.rsf, cfg.G, cfg.TG),
                               d.get("correction_bias"), d.get("expert_ids"))
    n_exp = distinct_experts(ids)
    l_bytes, l_flops = layer_algorithmic(cfg, n_exp)
    if backend == "staged":
        # the grouped gate_up GEMM with its fused activation dominates the layer
        log("[bench] timing the gate_up kernel")
        k_ms, _ = time_gate_up(cfg, d, args.kernel_reps)
        k_bytes = gate_up_algorithmic_bytes(cfg, n_exp)
        k_flops = gate_up_flops(cfg)
        k_name = "gemm_h16_kernel (grouped gate_up + SwiGLU)"
        k_traffic = recorded_traffic(cfg.name)
    else:
        # decode: the two indexed kernels stream the touched experts' weights; the
        # roofline entry covers one whole layer launch (route, permute, both indexed
        # kernels, combine) against the layer's minimum bytes
        log("[bench] timing the indexed layer")
        stream = torch.cuda.current_stream()
        k_ms = time_launches(lambda: run_layer(cfg, d, fcfg, ws, out, shared_out),
                             args.kernel_reps, stream)
        k_bytes = l_bytes
        k_flops = l_flops
        k_name = "moe_ffn_forward, indexed backend (indexed_kernel gate_up + down dominate)"
        k_traffic = recorded_traffic(cfg.name)
    # the binding roof of the timed kernel: MFMA above the ridge, HBM below it
    if k_flops / k_bytes > RIDGE:
        roof = {"bound": "mfma", "achieved": round(k_flops / (k_ms * 1e-3) / 1e12, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(k_bytes / (k_ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(float(np.median(step_ms)), 4),
                    "min": round(float(np.min(step_ms)), 4), "source": "HIP events per step"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs, random-init weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "F": cfg.F,
                   "top_k": cfg.K, "scoring": cfg.scoring, "activation": cfg.act,
                   "num_expert_group": cfg.G, "topk_group": cfg.TG, "F_shared": cfg.F_s,
                   "backend": backend, "parallelism": "single GPU"},
        "roofline": {**roof, "traffic": k_traffic, "kernel": k_name,
                     "kernel_ms": round(k_ms, 4), "algorithmic_bytes": k_bytes,
                     "algorithmic_flops": k_flops},
        "layer": {"hbm_frac": round(l_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(l_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                  "algorithmic_bytes": l_bytes, "flops": l_flops,
                  "distinct_experts": n_exp},
    }
    # the layer's fraction beside its target: 60 % of bf16 MFMA peak for prefill layers,
    # 70 % of HBM bandwidth for decode layers
    if backend == "staged":
        line["layer_mfma_frac"] = line["layer"]["mfma_frac"]
        line["mfma_target"] = 0.60
    else:
        line["layer_hbm_frac"] = line["layer"]["hbm_frac"]
        line["hbm_target"] = 0.70
    if not args.no_ceilings:
        log("[bench] measured ceilings")
        ceil = measured_ceilings()
        line["ceilings"] = ceil
        c = ceil["hbm_read_GBs"] if roof["unit"] == "GB/s" else ceil["mfma_bf16_TFLOPs"]
        line["roofline"]["measured_ceiling"] = c
        line["roofline"]["frac_of_measured_ceiling"] = round(roof["achieved"] / c, 4)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
