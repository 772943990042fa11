"""The whole layer (moe_ffn_forward) against the oracle's moe_ffn_forward().

Small shapes of each model family are compared on every token. The full-size workloads
are compared on a chosen set of tokens (every step of the layer is per token, so the
oracle can compute any subset): for every expert, the routes at the start and end of its
run in the expert-contiguous order and at every 32-row boundary inside it, so the first
and last rows of every row tile of every expert's GEMM tiles are compared. Routing is
compared on every token. A near-tie token (selection gap below 1e-6) must make a choice
the page's substitution rule allows; its output is then compared with the oracle's
output for that same choice (the oracle run with the GPU's expert ids)."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_ffn_moerouter_amd import binding as B
from mixture_experts_ffn_moerouter_amd import inputs as I
from moe_testlib import (LazyExperts, assert_close, check_route, near_tie_tokens, np64,
                         route_rerouter, say)

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
    # the decode backend's down contraction in chunks of 512: three here (and three passes
    # over one expert's routes in test_indexed_passes_over_route_groups), two below
    "decode_many_routes_per_expert": I.MoEConfig("decode_many", T=40, H=384, E=24, F=1536,
                                                 K=1, renormalize=False),
    "decode_like_indexed_chunks": I.MoEConfig("decode_like_indexed_chunks", T=16, H=256,
                                              E=64, F=1024, K=4, scoring="sigmoid", G=4, TG=2,
                                              correction_bias=(-0.1, 0.1), rsf=2.5),
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
    # float32 GEMMs large enough for the tiled kernel (the small float32 cases above take
    # the row-at-a-time one), with biases, groups and a shared expert
    "f32_tiled": I.MoEConfig("f32_tiled", T=512, H=256, E=8, F=128, K=2, dtype="f32",
                             scoring="sigmoid", G=4, TG=2, correction_bias=(-0.1, 0.1),
                             rsf=2.5, act="swigluoai", bias_std=0.1, w_std=0.05, F_s=128),
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
    # a shared expert of DeepSeek-V3-like size (M 4096, K 4096 and 2048, N 4096): every
    # token of its dense GEMMs compared, where the full-size layer test samples tokens
    "shared_dense_tiles": I.MoEConfig("shared_dense_tiles", T=4096, H=4096, E=8, F=64, K=2,
                                      F_s=2048),
}


def run_gpu(cfg, d, backend="auto"):
    """The layer on the GPU: (out, shared_out, topk_weights, topk_ids)."""
    w = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    ids = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    out, shared = B.moe_ffn_forward(
        B.ffn_cfg(cfg, backend), d["hidden"], d["logits"], d["w_gate_up"], d["w_down"],
        d.get("correction_bias"), d.get("expert_ids"), d.get("b_gate_up"), d.get("b_down"),
        d.get("shared_w_gate_up"), d.get("shared_w_down"), topk_weights_out=w,
        topk_ids_out=ids)
    return out, shared, w, ids


def run_oracle(cfg, d, tokens=None, expert_ids=None):
    """The oracle's layer on `tokens` (all by default). expert_ids, when given, is [n, K]
    for those tokens and replaces the routing choice (weights from those experts' scores)."""
    g = lambda k: None if d.get(k) is None else LazyExperts(d[k])
    sub = (lambda t: t) if tokens is None else (lambda t: t[tokens])
    if expert_ids is None and d.get("expert_ids") is not None:
        expert_ids = sub(d["expert_ids"]).cpu().numpy()
    return O.moe_ffn_forward(
        np64(sub(d["hidden"])), np64(sub(d["logits"])),
        LazyExperts(d["w_gate_up"]), LazyExperts(d["w_down"]), top_k=cfg.K,
        scoring=cfg.scoring, renormalize=cfg.renormalize, routed_scaling_factor=cfg.rsf,
        num_expert_group=cfg.G, topk_group=cfg.TG, act=cfg.act, dtype=cfg.dtype,
        correction_bias=None if d.get("correction_bias") is None else np64(d["correction_bias"]),
        expert_ids=expert_ids, b_gate_up=g("b_gate_up"), b_down=g("b_down"),
        shared_w_gate_up=None if d.get("shared_w_gate_up") is None else np64(d["shared_w_gate_up"]),
        shared_w_down=None if d.get("shared_w_down") is None else np64(d["shared_w_down"]))


def compare(cfg, d, out, shared, w_gpu, ids_gpu, tokens, what):
    """Every listed token: routing (ids, weights) and the layer output against the oracle;
    near-tie tokens against the oracle's layer for the GPU's own (valid) choice."""
    tokens = np.asarray(tokens)
    tt = torch.as_tensor(tokens, device="cuda")
    ref = run_oracle(cfg, d, tt)
    r = ref["route"]
    reroute = route_rerouter(np64(d["logits"][tt]), cfg.K, cfg.scoring, cfg.renormalize,
                             cfg.rsf)
    tie, _ = check_route(w_gpu[tt], ids_gpu[tt], r, what, reroute, cfg.G, cfg.TG)
    want = ref["out"]
    if tie.any():
        ti = np.nonzero(tie)[0]
        say(f"[ffn] {what}: {ti.size} near-tie token(s) compared on the GPU's choice")
        alt = run_oracle(cfg, d, torch.as_tensor(tokens[ti], device="cuda"),
                         expert_ids=ids_gpu[torch.as_tensor(tokens[ti], device="cuda")]
                         .cpu().numpy())
        want = want.copy()
        want[ti] = alt["out"]
    assert_close(np64(out)[tokens], want, cfg.dtype, what)
    if cfg.F_s:
        assert_close(np64(shared)[tokens], ref["shared_out"], cfg.dtype, what + " shared")
    return r


@pytest.mark.parametrize("name", sorted(SMALL))
def test_ffn_small(name):
    cfg = SMALL[name]
    say(f"[ffn] {name}")
    d = I.make_inputs(cfg, device="cuda")
    out, shared, w, ids = run_gpu(cfg, d)
    torch.cuda.synchronize()
    compare(cfg, d, out, shared, w, ids, np.arange(cfg.T), name)
    if name.startswith("decode"):
        assert B.moe_ffn_backend(B.ffn_cfg(cfg), False) == 2
        out_s = run_gpu(cfg, d, "staged")[0]
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
    out, shared, w, ids = run_gpu(cfg, d)
    torch.cuda.synchronize()
    r = compare(cfg, d, out, shared, w, ids, np.arange(cfg.T), "indexed 40 routes")
    assert (np.asarray(r.topk_ids) == 3).all()
    out_s = run_gpu(cfg, d, "staged")[0]
    torch.cuda.synchronize()
    assert_close(np64(out_s), np64(out), "bf16", "indexed vs staged")


def test_ffn_deterministic():
    cfg = SMALL["dsv3_like"]
    d = I.make_inputs(cfg, device="cuda")
    a = run_gpu(cfg, d)
    b = run_gpu(cfg, d)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_ffn_zero_tokens():
    cfg = SMALL["qwen_like"].with_(T=0)
    d = I.make_inputs(cfg, device="cuda")
    out = run_gpu(cfg, d)[0]
    assert out.shape == (0, 256)


# Full-size workloads: every output computed on the GPU; the tokens of coverage_tokens()
# compared with the oracle, the routing of every token.
FULL = ["tiny_fp32", "qwen3_bf16", "gptoss_bf16", "dsv3_bf16", "decode_dsv3_bf16",
        "qwen3_skewed_bf16", "qwen3_f16", "qwen3_gelu_bf16"]


def coverage_tokens(topk_ids: np.ndarray, E: int, stride: int = 32) -> np.ndarray:
    """Tokens whose routes sit, in the expert-contiguous (stable, route-ordered) layout,
    at the first and last row of every expert's run and on both sides of every
    `stride`-row boundary inside it: any row tile whose height is a multiple of `stride`
    has its first and last row among them."""
    off, srt, _ = O.permute(topk_ids, E)
    K = topk_ids.shape[1]
    pos = []
    for e in range(E):
        m = int(off[e + 1] - off[e])
        if m == 0:
            continue
        j = np.arange(stride, m, stride)
        pos.append(off[e] + np.unique(np.concatenate([[0, m - 1], j - 1, j])))
    return np.unique(srt[np.concatenate(pos)] // K)


@pytest.mark.parametrize("name", FULL)
def test_ffn_full_size_every_expert(name):
    cfg = I.CONFIGS[name]
    say(f"[ffn-full] {name} generating inputs")
    d = I.make_inputs(cfg, device="cuda")
    say(f"[ffn-full] {name} forward")
    out, shared, w, ids = run_gpu(cfg, d)
    torch.cuda.synchronize()
    # routing of every token (the topk copies the layer returned)
    lg = np64(d["logits"])
    cb = None if d.get("correction_bias") is None else np64(d["correction_bias"])
    r = O.route(lg, cfg.K, cfg.scoring, cfg.renormalize, cfg.rsf, cfg.G, cfg.TG, cb)
    check_route(w, ids, r, name, route_rerouter(lg, cfg.K, cfg.scoring, cfg.renormalize,
                                                cfg.rsf), cfg.G, cfg.TG)
    tokens = coverage_tokens(r.topk_ids, cfg.E)
    experts = np.unique(r.topk_ids[tokens])
    used = np.unique(r.topk_ids)
    assert np.array_equal(experts, used), "an expert's rows are not covered"
    say(f"[ffn-full] {name}: oracle on {tokens.size} tokens covering all {used.size} "
        f"routed experts")
    compare(cfg, d, out, shared, w, ids, tokens, name)
    assert np.all(np.isfinite(np64(out)))
    del d
    torch.cuda.empty_cache()
