"""The whole layer (moe_ffn_forward) against the oracle's moe_ffn_forward().

Small shapes of each model family are compared on every token; the full-size workloads
are compared on sampled tokens (the oracle computes one token at a time, and every step
of the layer is per token). Tokens whose routing is a near tie are left out of the
output comparison; their routing is checked for validity instead."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_ffn_moerouter_amd import binding as B
from mixture_experts_ffn_moerouter_amd import inputs as I
from moe_testlib import LazyExperts, assert_close, check_route, np64, say

pytestmark = pytest.mark.gpu

SMALL = {
    "qwen_like": I.MoEConfig("qwen_like", T=300, H=256, E=16, F=192, K=4),
    "gptoss_like": I.MoEConfig("gptoss_like", T=200, H=200, E=8, F=96, K=4, act="swigluoai",
                               bias_std=0.3, x_std=4.0, w_std=0.1),
    "dsv3_like": I.MoEConfig("dsv3_like", T=256, H=512, E=32, F=128, K=8, scoring="sigmoid",
                             rsf=2.5, G=8, TG=4, correction_bias=(-0.1, 0.1), F_s=192),
    "hash_sqrt_softplus": I.MoEConfig("hash_sqrt_softplus", T=128, H=128, E=24, F=64, K=3,
                                      scoring="sqrt_softplus", hash_routing=True),
    "tiny_fp32_groups": I.MoEConfig("tiny_fp32_groups", T=70, H=96, E=12, F=40, K=3,
                                    dtype="f32", scoring="sigmoid", G=4, TG=2,
                                    correction_bias=(-0.1, 0.1), F_s=24, rsf=1.7,
                                    act="swigluoai", bias_std=0.1, w_std=0.1),
    "decode_like_indexed": I.MoEConfig("decode_like_indexed", T=16, H=256, E=64, F=256, K=4,
                                       scoring="sigmoid", G=4, TG=2,
                                       correction_bias=(-0.1, 0.1), rsf=2.5),
    "decode_many_routes_per_expert": I.MoEConfig("decode_many", T=40, H=384, E=24, F=512,
                                                 K=1, renormalize=False),
    "single_token": I.MoEConfig("single_token", T=1, H=128, E=4, F=64, K=2),
    # a per-expert logit ramp: some experts take most tokens, many take none
    "skewed_load": I.MoEConfig("skewed_load", T=600, H=320, E=48, F=192, K=6, logit_skew=6.0),
    # float16 operands (staged and indexed), gelu_and_mul, 16-bit router logits
    "qwen_like_f16": I.MoEConfig("qwen_like_f16", T=300, H=256, E=16, F=192, K=4, dtype="f16"),
    "gptoss_like_f16": I.MoEConfig("gptoss_like_f16", T=200, H=200, E=8, F=96, K=4,
                                   act="swigluoai", bias_std=0.3, x_std=4.0, w_std=0.1,
                                   dtype="f16"),
    "decode_like_indexed_f16": I.MoEConfig("decode_like_indexed_f16", T=16, H=256, E=64,
                                           F=256, K=4, scoring="sigmoid", G=4, TG=2,
                                           correction_bias=(-0.1, 0.1), rsf=2.5, dtype="f16"),
    "gelu_like": I.MoEConfig("gelu_like", T=300, H=256, E=16, F=192, K=4, act="gelu_and_mul",
                             x_std=2.0, w_std=0.1),
    "gelu_like_f32": I.MoEConfig("gelu_like_f32", T=70, H=96, E=12, F=40, K=3, dtype="f32",
                                 act="gelu_and_mul", bias_std=0.1, w_std=0.1),
    "bf16_logits_groups": I.MoEConfig("bf16_logits_groups", T=256, H=512, E=32, F=128, K=8,
                                      scoring="sigmoid", rsf=2.5, G=8, TG=4,
                                      correction_bias=(-0.1, 0.1), logits_dtype="bf16"),
    "f16_logits_softmax": I.MoEConfig("f16_logits_softmax", T=300, H=256, E=16, F=192, K=4,
                                      logits_dtype="f16"),
    # E at the router's maximum of 512, through each backend
    "max_experts_staged": I.MoEConfig("max_experts_staged", T=400, H=128, E=512, F=64, K=8,
                                      scoring="sigmoid", G=8, TG=4,
                                      correction_bias=(-0.1, 0.1), rsf=2.5),
    "decode_max_experts": I.MoEConfig("decode_max_experts", T=64, H=128, E=512, F=256, K=8,
                                      scoring="sigmoid", G=8, TG=4,
                                      correction_bias=(-0.1, 0.1), rsf=2.5),
}


def run_gpu(cfg, d, backend="auto"):
    out, shared = B.moe_ffn_forward(
        B.ffn_cfg(cfg, backend), d["hidden"], d["logits"], d["w_gate_up"], d["w_down"],
        d.get("correction_bias"), d.get("expert_ids"), d.get("b_gate_up"), d.get("b_down"),
        d.get("shared_w_gate_up"), d.get("shared_w_down"),
        topk_weights_out=torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda"),
        topk_ids_out=torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda"))
    return out, shared


def run_oracle(cfg, d, tokens=None):
    g = lambda k: None if d.get(k) is None else LazyExperts(d[k])
    return O.moe_ffn_forward(
        np64(d["hidden"]) if tokens is None else np64(d["hidden"][tokens]),
        np64(d["logits"]) if tokens is None else np64(d["logits"][tokens]),
        LazyExperts(d["w_gate_up"]), LazyExperts(d["w_down"]), top_k=cfg.K,
        scoring=cfg.scoring, renormalize=cfg.renormalize, routed_scaling_factor=cfg.rsf,
        num_expert_group=cfg.G, topk_group=cfg.TG, act=cfg.act, dtype=cfg.dtype,
        correction_bias=None if d.get("correction_bias") is None else np64(d["correction_bias"]),
        expert_ids=None if d.get("expert_ids") is None else (
            d["expert_ids"].cpu().numpy() if tokens is None
            else d["expert_ids"][tokens].cpu().numpy()),
        b_gate_up=g("b_gate_up"), b_down=g("b_down"),
        shared_w_gate_up=None if d.get("shared_w_gate_up") is None else np64(d["shared_w_gate_up"]),
        shared_w_down=None if d.get("shared_w_down") is None else np64(d["shared_w_down"]))


def compare(cfg, d, out, shared, tokens, what):
    tokens = np.asarray(tokens)
    ref = run_oracle(cfg, d, torch.as_tensor(tokens, device="cuda"))
    r = ref["route"]
    # routing: the topk copies moe_ffn_forward returned
    tie = np.asarray(r.gap_sel < 1e-6) | np.asarray(r.gap_group < 1e-6)
    ok = ~tie
    got = np64(out)[tokens]
    assert_close(got[ok], ref["out"][ok], cfg.dtype, what)
    if cfg.F_s:
        assert_close(np64(shared)[tokens], ref["shared_out"], cfg.dtype, what + " shared")
    return r


@pytest.mark.parametrize("name", sorted(SMALL))
def test_ffn_small(name):
    cfg = SMALL[name]
    say(f"[ffn] {name}")
    d = I.make_inputs(cfg, device="cuda")
    out, shared = run_gpu(cfg, d)
    torch.cuda.synchronize()
    compare(cfg, d, out, shared, np.arange(cfg.T), name)
    if name.startswith("decode"):
        assert B.moe_ffn_backend(B.ffn_cfg(cfg), False) == 2
        out_s, _ = run_gpu(cfg, d, "staged")
        torch.cuda.synchronize()
        assert_close(np64(out_s), np64(out), cfg.dtype, "indexed vs staged")


def test_indexed_passes_over_route_groups():
    """One expert takes every route (40 > 16), so the decode backend runs three passes of
    16, 16 and 8 routes over that expert's weights."""
    cfg = SMALL["decode_many_routes_per_expert"]
    say("[ffn] indexed, 40 routes on one expert")
    d = I.make_inputs(cfg, device="cuda")
    d["logits"][:, 3] += 30.0
    assert B.moe_ffn_backend(B.ffn_cfg(cfg), False) == 2
    out, shared = run_gpu(cfg, d)
    torch.cuda.synchronize()
    r = compare(cfg, d, out, shared, np.arange(cfg.T), "indexed 40 routes")
    assert (np.asarray(r.topk_ids) == 3).all()
    out_s, _ = run_gpu(cfg, d, "staged")
    torch.cuda.synchronize()
    assert_close(np64(out_s), np64(out), "bf16", "indexed vs staged")


def test_ffn_deterministic():
    cfg = SMALL["dsv3_like"]
    d = I.make_inputs(cfg, device="cuda")
    a = run_gpu(cfg, d)
    b = run_gpu(cfg, d)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_ffn_zero_tokens():
    cfg = SMALL["qwen_like"].with_(T=0)
    d = I.make_inputs(cfg, device="cuda")
    out, _ = run_gpu(cfg, d)
    assert out.shape == (0, 256)


# Full-size workloads: every output computed on the GPU, sampled tokens checked.
FULL = ["tiny_fp32", "qwen3_bf16", "gptoss_bf16", "dsv3_bf16", "decode_dsv3_bf16",
        "qwen3_skewed_bf16", "qwen3_f16", "qwen3_gelu_bf16"]
SAMPLES = {"tiny_fp32": 64, "qwen3_bf16": 12, "gptoss_bf16": 8, "dsv3_bf16": 4,
           "decode_dsv3_bf16": 6, "qwen3_skewed_bf16": 8, "qwen3_f16": 12,
           "qwen3_gelu_bf16": 12}


@pytest.mark.parametrize("name", FULL)
def test_ffn_full_size(name):
    cfg = I.CONFIGS[name]
    say(f"[ffn-full] {name} generating inputs")
    d = I.make_inputs(cfg, device="cuda")
    say(f"[ffn-full] {name} forward")
    out, shared = run_gpu(cfg, d)
    torch.cuda.synchronize()
    n = SAMPLES[name]
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(cfg.T, size=min(n, cfg.T), replace=False))
    say(f"[ffn-full] {name} oracle on tokens {tokens.tolist()}")
    compare(cfg, d, out, shared, tokens, name)
    # routing of every token, through moe_route (same kernel moe_ffn_forward runs)
    w, ids, _, _ = B.moe_route(d["logits"], B.route_cfg(cfg.K, cfg.scoring, cfg.renormalize,
                                                        cfg.rsf, cfg.G, cfg.TG),
                               d.get("correction_bias"))
    torch.cuda.synchronize()
    r = O.route(np64(d["logits"]), cfg.K, cfg.scoring, cfg.renormalize, cfg.rsf, cfg.G,
                cfg.TG, None if d.get("correction_bias") is None else np64(d["correction_bias"]))
    check_route(w, ids, r, name)
    # properties at every token: finite, and a bf16 output bounded like the sample
    o = np64(out)
    assert np.all(np.isfinite(o))
    del d
    torch.cuda.empty_cache()
