"""Seeded synthetic inputs for the routed MoE FFN: workload shapes and generators.

This module holds none of the method's arithmetic. It feeds the same tensors to the GPU
library and to the CPU oracle, so it imports neither.

Generator: a counter-based SplitMix64 stream (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014: state step 0x9E3779B97F4A7C15 and the
"mix64" finaliser with multipliers 0xBF58476D1CE4E5B9 / 0x94D049BB133111EB). Element i
of the tensor with stream id `stream` under `seed` takes the 64-bit word
    mix64(key + (c + 1) * 0x9E3779B97F4A7C15),   key = mix64(seed * 0x9E3779B97F4A7C15 + stream)
for counter c; the top 53 bits give a uniform u in [0, 1). Normals use the Box-Muller
transform (Box and Muller, 1958) on counters 2i and 2i+1:
    n = sqrt(-2 ln(1 - u_2i)) * cos(2 pi u_2i+1).
Values are computed in float64 and then cast to the tensor dtype. Any element can be
regenerated alone, and torch integer ops wrap identically on CPU and GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 24

# Stream id of every generated tensor.
STREAMS = {
    "hidden": 0, "logits": 1, "w_gate_up": 2, "w_down": 3, "b_gate_up": 4, "b_down": 5,
    "correction_bias": 6, "shared_w_gate_up": 7, "shared_w_down": 8, "expert_ids": 9,
    "fp8_a": 10, "fp8_b": 11, "fp8_counts": 12,
}


def _s64(v: int) -> int:
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (reference for the tensor version)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def _shr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)  # logical shift of an int64 tensor


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _shr(z, 30)) * _s64(_M1)
    z = (z ^ _shr(z, 27)) * _s64(_M2)
    return z ^ _shr(z, 31)


def stream_key(seed: int, stream: int) -> int:
    return mix64_int(seed * _GOLDEN + stream)


def uniform_words(key: int, counters: torch.Tensor) -> torch.Tensor:
    """64-bit words (as int64) of the stream at the given int64 counters."""
    return _mix64(_s64(key) + (counters + 1) * _s64(_GOLDEN))


def _uniform(key: int, counters: torch.Tensor) -> torch.Tensor:
    return _shr(uniform_words(key, counters), 11).to(torch.float64) * (2.0 ** -53)


def _fill(out: torch.Tensor, key: int, kind: str, a: float, b: float,
          start: int = 0) -> torch.Tensor:
    flat = out.view(-1)
    n = flat.numel()
    dev = out.device
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        i = torch.arange(start + lo, start + hi, dtype=torch.int64, device=dev)
        if kind == "normal":
            u1 = _uniform(key, 2 * i)
            u2 = _uniform(key, 2 * i + 1)
            v = torch.sqrt(-2.0 * torch.log1p(-u1)) * torch.cos((2.0 * math.pi) * u2)
            v = a + b * v
        elif kind == "uniform":
            v = a + (b - a) * _uniform(key, i)
        else:
            raise ValueError(kind)
        flat[lo:hi] = v.to(out.dtype)
    return out


def normal(shape, std: float, *, seed: int, stream: int, dtype=torch.float32,
           device="cpu", mean: float = 0.0, start: int = 0) -> torch.Tensor:
    """Elements start, start+1, ... of the stream (start lets a large tensor be made in
    pieces that equal the corresponding slices of the whole)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    return _fill(out, stream_key(seed, stream), "normal", mean, std, start)


def uniform(shape, lo: float, hi: float, *, seed: int, stream: int, dtype=torch.float32,
            device="cpu") -> torch.Tensor:
    out = torch.empty(shape, dtype=dtype, device=device)
    return _fill(out, stream_key(seed, stream), "uniform", lo, hi)


def random_expert_ids(T: int, K: int, E: int, *, seed: int, device="cpu") -> torch.Tensor:
    """[T,K] int32 hash-routing ids, K distinct experts per token (a seeded permutation)."""
    key = stream_key(seed, STREAMS["expert_ids"])
    i = torch.arange(T * E, dtype=torch.int64, device=device)
    r = _shr(uniform_words(key, i), 1).view(T, E)
    return torch.argsort(r, dim=1)[:, :K].to(torch.int32)


_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class MoEConfig:
    """One workload: model shapes, routing and activation options, input distributions."""
    name: str
    T: int
    H: int
    E: int
    F: int
    K: int
    scoring: str = "softmax"
    renormalize: bool = True
    rsf: float = 1.0
    G: int = 1
    TG: int = 1
    act: str = "silu_and_mul"
    dtype: str = "bf16"
    w_std: float = 0.02
    x_std: float = 1.0
    logit_std: float = 1.0
    bias_std: Optional[float] = None            # b_gate_up / b_down ~ N(0, bias_std)
    correction_bias: Optional[tuple] = None     # (lo, hi) uniform
    F_s: int = 0                                # shared expert width; 0 = none
    local_expert_start: int = 0
    local_expert_count: Optional[int] = None
    router_probs_dtype: Optional[str] = None
    hash_routing: bool = False
    logit_skew: float = 0.0                     # logits[:, e] += logit_skew * e / (E - 1)
    logits_dtype: str = "f32"                   # storage of the router logits
    notes: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        return self.T * self.K

    @property
    def torch_dtype(self):
        return _TORCH_DT[self.dtype]

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


# The workloads. Shapes follow the model families the pages name: Qwen3 softmax
# routing; gpt-oss interleaved swigluoai with expert biases; DeepSeek-V3 sigmoid routing
# with correction bias, 8 groups / 4 kept, scaling 2.5 and a shared expert.
CONFIGS = {
    "tiny_fp32": MoEConfig("tiny_fp32", T=64, H=128, E=8, F=64, K=2, dtype="f32",
                           w_std=0.05),
    "qwen3_bf16": MoEConfig("qwen3_bf16", T=4096, H=2048, E=128, F=768, K=8),
    "gptoss_bf16": MoEConfig("gptoss_bf16", T=2048, H=2880, E=128, F=2880, K=4,
                             act="swigluoai", bias_std=0.01),
    "dsv3_bf16": MoEConfig("dsv3_bf16", T=4096, H=7168, E=256, F=2048, K=8,
                           scoring="sigmoid", rsf=2.5, G=8, TG=4,
                           correction_bias=(-0.1, 0.1), F_s=2048),
    # Compute-bound evidence point (not a graded workload): the Qwen3 shapes at four times
    # the tokens, ~1024 routes per expert, arithmetic intensity above the ridge.
    "qwen3_bf16_t16k": MoEConfig("qwen3_bf16_t16k", T=16384, H=2048, E=128, F=768, K=8),
    # Skewed expert load (a per-expert logit offset): a few experts take most tokens.
    "qwen3_skewed_bf16": MoEConfig("qwen3_skewed_bf16", T=4096, H=2048, E=128, F=768, K=8,
                                   logit_skew=6.0),
    # The Qwen3 shapes with float16 operands, and with gelu_and_mul (the next rows' dtype
    # and activation on the bench workload's shapes).
    "qwen3_f16": MoEConfig("qwen3_f16", T=4096, H=2048, E=128, F=768, K=8, dtype="f16"),
    "qwen3_gelu_bf16": MoEConfig("qwen3_gelu_bf16", T=4096, H=2048, E=128, F=768, K=8,
                                 act="gelu_and_mul"),
    "decode_dsv3_bf16": MoEConfig("decode_dsv3_bf16", T=16, H=7168, E=256, F=2048, K=8,
                                  scoring="sigmoid", rsf=2.5, G=8, TG=4,
                                  correction_bias=(-0.1, 0.1)),
    # Router-only pass: sqrt_softplus scoring, plain top-k, one expert-parallel slice.
    "router_ep_f16": MoEConfig("router_ep_f16", T=16, H=0, E=256, F=0, K=8,
                               scoring="sqrt_softplus", local_expert_start=64,
                               local_expert_count=64, router_probs_dtype="f16"),
    # Router-only pass at prefill size with bfloat16 logits: the DeepSeek-V3 router
    # (sigmoid, correction bias, 8 groups / 4 kept, top-8, scaling 2.5).
    "router_dsv3_bf16_logits": MoEConfig("router_dsv3_bf16_logits", T=4096, H=0, E=256, F=0,
                                         K=8, scoring="sigmoid", rsf=2.5, G=8, TG=4,
                                         correction_bias=(-0.1, 0.1), logits_dtype="bf16"),
}


def make_router_inputs(cfg: MoEConfig, *, seed: int = 0, device="cpu") -> dict:
    d = {"logits": normal((cfg.T, cfg.E), cfg.logit_std, seed=seed,
                          stream=STREAMS["logits"], dtype=torch.float32, device=device)}
    if cfg.logit_skew:
        ramp = torch.arange(cfg.E, dtype=torch.float32, device=device) / max(cfg.E - 1, 1)
        d["logits"] += cfg.logit_skew * ramp
    if cfg.correction_bias is not None:
        lo, hi = cfg.correction_bias
        d["correction_bias"] = uniform((cfg.E,), lo, hi, seed=seed,
                                       stream=STREAMS["correction_bias"],
                                       dtype=torch.float32, device=device)
    if cfg.hash_routing:
        d["expert_ids"] = random_expert_ids(cfg.T, cfg.K, cfg.E, seed=seed, device=device)
    if cfg.logits_dtype != "f32":
        d["logits"] = d["logits"].to(_TORCH_DT[cfg.logits_dtype])
    return d


def make_inputs(cfg: MoEConfig, *, seed: int = 0, device="cpu") -> dict:
    """All input tensors of one workload, generated directly on `device`."""
    dt = cfg.torch_dtype
    d = make_router_inputs(cfg, seed=seed, device=device)
    d["hidden"] = normal((cfg.T, cfg.H), cfg.x_std, seed=seed, stream=STREAMS["hidden"],
                         dtype=dt, device=device)
    d["w_gate_up"] = normal((cfg.E, 2 * cfg.F, cfg.H), cfg.w_std, seed=seed,
                            stream=STREAMS["w_gate_up"], dtype=dt, device=device)
    d["w_down"] = normal((cfg.E, cfg.H, cfg.F), cfg.w_std, seed=seed,
                         stream=STREAMS["w_down"], dtype=dt, device=device)
    if cfg.bias_std is not None:
        d["b_gate_up"] = normal((cfg.E, 2 * cfg.F), cfg.bias_std, seed=seed,
                                stream=STREAMS["b_gate_up"], dtype=dt, device=device)
        d["b_down"] = normal((cfg.E, cfg.H), cfg.bias_std, seed=seed,
                             stream=STREAMS["b_down"], dtype=dt, device=device)
    if cfg.F_s:
        d["shared_w_gate_up"] = normal((2 * cfg.F_s, cfg.H), cfg.w_std, seed=seed,
                                       stream=STREAMS["shared_w_gate_up"], dtype=dt,
                                       device=device)
        d["shared_w_down"] = normal((cfg.H, cfg.F_s), cfg.w_std, seed=seed,
                                    stream=STREAMS["shared_w_down"], dtype=dt,
                                    device=device)
    return d


# --------------------------------------------------------------------------------------
# Block-scaled FP8 grouped GEMM over a masked slab (a [E, max_m, K], b [E, N, K]).

@dataclass(frozen=True)
class Fp8GemmConfig:
    """One FP8 masked grouped GEMM workload. counts, when given, fixes the valid rows of
    each expert; otherwise they are round(N(rows_mean, rows_std)) clamped to [0, max_m]."""
    name: str
    E: int
    max_m: int
    K: int
    N: int
    rows_mean: float = 0.0
    rows_std: float = 0.0
    counts: Optional[tuple] = None
    a_std: float = 1.0
    b_std: float = 0.02
    notes: str = field(default="", compare=False)


FP8_CONFIGS = {
    # small parity case: empty, single-row, ragged, full and over-full experts
    "fp8_small": Fp8GemmConfig("fp8_small", E=7, max_m=160, K=384, N=384,
                               counts=(0, 1, 37, 128, 129, 160, 200)),
    # the DeepSeek-V3 routed expert GEMMs in the masked layout: about 128 routes per
    # expert (T 4096, top-8 of 256), slabs of 256 rows
    "dsv3_fp8_gate_up": Fp8GemmConfig("dsv3_fp8_gate_up", E=256, max_m=256, K=7168, N=4096,
                                      rows_mean=128.0, rows_std=11.1),
    "dsv3_fp8_down": Fp8GemmConfig("dsv3_fp8_down", E=256, max_m=256, K=2048, N=7168,
                                   rows_mean=128.0, rows_std=11.1),
}


def _quantize_e4m3fn_blocks(x: torch.Tensor, rows_per_block: int):
    """x [R, K] float32 -> (codes [R, K] uint8, scales [R/rows_per_block, K/128] float32):
    each rows_per_block x 128 block is divided by amax/448 (1 for an all-zero block) and
    cast to float8_e4m3fn (round to nearest even)."""
    R, K = x.shape
    xb = x.view(R // rows_per_block, rows_per_block, K // 128, 128)
    amax = xb.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (xb / scale[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(R, K).view(torch.uint8), scale.to(torch.float32)


def make_fp8_inputs(cfg: Fp8GemmConfig, *, seed: int = 0, device="cpu") -> dict:
    """a, a_scale, b, b_scale (codes as uint8) and counts of one FP8 workload, generated
    one expert at a time."""
    E, M, K, N = cfg.E, cfg.max_m, cfg.K, cfg.N
    a = torch.empty((E, M, K), dtype=torch.uint8, device=device)
    b = torch.empty((E, N, K), dtype=torch.uint8, device=device)
    sa = torch.empty((E, M, K // 128), dtype=torch.float32, device=device)
    sb = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=device)
    for g in range(E):
        xa = normal((M, K), cfg.a_std, seed=seed, stream=STREAMS["fp8_a"], device=device,
                    start=g * M * K)
        a[g], sa[g] = _quantize_e4m3fn_blocks(xa, 1)
        xb = normal((N, K), cfg.b_std, seed=seed, stream=STREAMS["fp8_b"], device=device,
                    start=g * N * K)
        b[g], sb[g] = _quantize_e4m3fn_blocks(xb, 128)
    return {"a": a, "a_scale": sa, "b": b, "b_scale": sb,
            "counts": fp8_counts(cfg, seed=seed, device=device)}


def fp8_counts(cfg: Fp8GemmConfig, *, seed: int = 0, device="cpu") -> torch.Tensor:
    """Valid rows per expert of an FP8 workload: cfg.counts, or round(N(rows_mean,
    rows_std)) clamped to [0, max_m]."""
    if cfg.counts is not None:
        return torch.tensor(cfg.counts, dtype=torch.int32, device=device)
    c = normal((cfg.E,), cfg.rows_std, seed=seed, stream=STREAMS["fp8_counts"],
               dtype=torch.float64, device=device, mean=cfg.rows_mean)
    return c.round().clamp(0, cfg.max_m).to(torch.int32)


# --------------------------------------------------------------------------------------
# Standalone SwiGLU operator ([MR] SwiGLU): one fused [rows, 2F] projection in, [rows, F]
# out.

@dataclass(frozen=True)
class SwigluConfig:
    name: str
    rows: int
    F: int
    dtype: str = "bf16"
    fusion: str = "stacked"        # gate then up ([MR], up omitted)
    alpha: float = 1.702
    beta: float = 1.0
    limit: float = 7.0
    x_std: float = 4.0             # the clamps fire at |x| > 7


SWIGLU_CONFIGS = {
    # The [MR] case: a tensor-parallel shared expert's fused gate_up output (16384 tokens x
    # 2 x 4096), the gpt-oss constants.
    "swiglu_bf16": SwigluConfig("swiglu_bf16", rows=16384, F=4096),
    "swiglu_small": SwigluConfig("swiglu_small", rows=37, F=96, dtype="f16",
                                 fusion="interleaved"),
}


def make_swiglu_inputs(cfg: SwigluConfig, *, seed: int = 0, device="cpu") -> dict:
    """The fused projection: STREAMS["hidden"] values at x_std, [rows, 2F]."""
    return {"gate": normal((cfg.rows, 2 * cfg.F), cfg.x_std, seed=seed,
                           stream=STREAMS["hidden"], dtype=_TORCH_DT[cfg.dtype],
                           device=device)}


# --------------------------------------------------------------------------------------
# Layout workloads ([TO] MoEPrePermuteFwdOp, MoEGroupedGemmFwdOp's masked layout).

@dataclass(frozen=True)
class LayoutConfig:
    name: str
    kind: str                      # "pre_permute" or "masked_gemm"
    route: Optional[str] = None    # pre_permute: the MoEConfig whose routing it permutes
    layout: str = "contiguous"
    block_size: int = 64
    fp8: Optional[str] = None      # masked_gemm: the Fp8GemmConfig whose shapes it takes
    w_std: float = 0.02


LAYOUT_CONFIGS = {
    # Qwen3 routing (T 4096, top-8 of 128) into block-aligned expert rows, block 64.
    "qwen3_pre_permute_bs64": LayoutConfig("qwen3_pre_permute_bs64", "pre_permute",
                                           route="qwen3_bf16"),
    # The DeepSeek-V3 gate_up shape over a masked slab, in bfloat16 (the FP8 workload's
    # shapes and counts).
    "dsv3_bf16_masked_gate_up": LayoutConfig("dsv3_bf16_masked_gate_up", "masked_gemm",
                                             layout="masked", fp8="dsv3_fp8_gate_up"),
}
