"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

A pin suite that still passes with a mistake planted would not be pinning that part.
"""
import math

import numpy as np
import pytest

import oracle.moe_oracle as O
import oracle_pins as P


def _swiglu_two_sided_gate(g, l, alpha=1.0, beta=0.0, limit=0.0):
    g = np.asarray(g, np.float64)
    l = np.asarray(l, np.float64)
    if limit > 0:
        g = np.clip(g, -limit, limit)
        l = np.clip(l, -limit, limit)
    return g * O.sigmoid(alpha * g) * (l + beta)


def _swiglu_no_disable(g, l, alpha=1.0, beta=0.0, limit=0.0):
    g = np.minimum(np.asarray(g, np.float64), limit if limit > 0 else 7.0)
    l = np.clip(np.asarray(l, np.float64), -7.0, 7.0) if limit <= 0 else np.clip(l, -limit, limit)
    return g * O.sigmoid(alpha * g) * (l + beta)


def _split_swapped(h, layout):
    g, u = _orig_split(h, layout)
    return u, g


def _ranked_high_index(values):
    v = np.asarray(values, np.float64)
    return np.lexsort((-np.arange(v.size), -v))


def _weights_rsf_twice(s, sel, renormalize, rsf):
    wn, w = _orig_weights(s, sel, renormalize, rsf)
    return wn, w * rsf


def _weights_biased(s, sel, renormalize, rsf):
    # renormalize by the sum over all experts instead of the chosen ones
    w = np.take_along_axis(np.asarray(s, np.float64), np.asarray(sel), axis=1)
    wn = w / np.asarray(s).sum(axis=1, keepdims=True) if renormalize else w
    return wn, wn * rsf


def _combine_transposed(y, topk_weights, route_pos, scale=1.0, out_dtype="f32"):
    w = np.asarray(topk_weights, np.float64)
    T, K = w.shape
    pos = np.asarray(route_pos).reshape(K, T).T
    out = np.zeros((T, np.asarray(y).shape[1]))
    for k in range(K):
        out += w[:, k:k + 1] * np.asarray(y)[pos[:, k]]
    return O.round_to(scale * out, out_dtype)


def _expert_mlp_unrounded_act(x, w_gate_up, w_down, b_gate_up=None, b_down=None,
                              act="silu_and_mul", act_dtype="f32"):
    return _orig_expert_mlp(x, w_gate_up, w_down, b_gate_up, b_down, act, "f64")


def _expert_mlp_no_down_bias(x, w_gate_up, w_down, b_gate_up=None, b_down=None,
                             act="silu_and_mul", act_dtype="f32"):
    return _orig_expert_mlp(x, w_gate_up, w_down, b_gate_up, None, act, act_dtype)


def _round_truncate(x, fmt):
    x = np.asarray(x, np.float64)
    if fmt == "f64":
        return x.copy()
    p, emin, emax = O.FORMATS[fmt]
    out = x.copy()
    m = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[m])
    ue = np.maximum(e - p, emin - p + 1)
    out[m] = np.ldexp(np.trunc(np.ldexp(x[m], -ue)), ue)
    return out


def _scores_sqrt_softplus_wrong(logits, scoring):
    if scoring == "sqrt_softplus":
        z = np.asarray(logits, np.float64)
        return np.sqrt(np.log1p(np.exp(-np.abs(z))))   # dropped max(z, 0) term
    return _orig_scores(logits, scoring)


def _group_max_with_bias(s, top_k, correction_bias=None, num_expert_group=1, topk_group=1):
    # group score = best biased score instead of the sum of the two best
    if correction_bias is None:
        return _orig_select(s, top_k, None, num_expert_group, topk_group)
    s32 = O.round_to(s, "f32")
    T, E = s32.shape
    u = O.round_to(s32 + np.asarray(correction_bias)[None], "f32")
    G, TG = num_expert_group, topk_group
    sel = np.zeros((T, top_k), np.int64)
    for t in range(T):
        elig = np.ones(E, bool)
        if G > 1:
            gs = u[t].reshape(G, -1).max(1)
            elig = np.isin(np.arange(E) // (E // G), O.ranked(gs)[:TG])
        cand = np.nonzero(elig)[0]
        sel[t] = cand[O.ranked(u[t, cand])][:top_k]
    return sel, np.full(T, np.inf), np.full(T, np.inf)


def _permute_unstable(topk_ids, num_experts):
    off, srt, pos = _orig_permute(topk_ids, num_experts)
    srt = srt.copy()
    for e in range(num_experts):
        srt[off[e]:off[e + 1]] = srt[off[e]:off[e + 1]][::-1]
    pos = np.empty_like(srt)
    pos[srt] = np.arange(srt.size)
    return off, srt, pos


def _ep_fill_everywhere_zero_scale(sel, wn, rsf, start, count, dtype):
    rp, ws = _orig_ep(sel, wn, rsf, start, count, dtype)
    return rp, np.where(ws == 0, O.round_to(rsf, dtype), ws)


_orig_split = O.split_gate_up
_orig_weights = O.routing_weights
_orig_expert_mlp = O.expert_mlp
_orig_scores = O.scores
_orig_select = O.select_experts
_orig_permute = O.permute
_orig_ep = O.ep_router_outputs

_orig_fp8 = O.grouped_gemm_fp8_masked
_orig_decode = O.decode_e4m3fn


def _decode_fnuz(codes):
    # the other FP8 E4M3 encoding (exponent bias 8)
    return _orig_decode(codes) / 2.0


def _fp8_block_scale_tiled(a_codes, a_scale, b_codes, b_scale, counts):
    # b_scale expanded along n by tiling (n % blocks) instead of n // 128
    A = O.decode_e4m3fn(a_codes)
    B = O.decode_e4m3fn(b_codes)
    E, max_m, K = A.shape
    N = B.shape[1]
    out = np.full((E, max_m, N), np.nan)
    for g in range(E):
        m = int(min(max(int(counts[g]), 0), max_m))
        acc = np.zeros((m, N))
        for kb in range(K // 128):
            ks = slice(128 * kb, 128 * (kb + 1))
            acc += (A[g, :m, ks] @ B[g, :, ks].T) * a_scale[g, :m, kb][:, None] * \
                np.tile(b_scale[g, :, kb], 128)[None, :N]
        out[g, :m] = O.round_to(acc, "bf16")
    return out


def _fp8_counts_unclamped(a_codes, a_scale, b_codes, b_scale, counts):
    return _orig_fp8(a_codes, a_scale, b_codes, b_scale, np.abs(np.asarray(counts)))


def _fp8_no_a_scale(a_codes, a_scale, b_codes, b_scale, counts):
    return _orig_fp8(a_codes, np.ones_like(np.asarray(a_scale)), b_codes, b_scale, counts)


_orig_gated = O.gated
_orig_swiglu_op = O.swiglu_op


def _gelu_tanh(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def _gated_act_on_up(g, l, params):
    if params[4] == "gelu":
        return np.asarray(g, dtype=np.float64) * O.gelu(l)
    return _orig_gated(g, l, params)


def _swiglu_op_ignores_fusion(gate, up=None, alpha=1.0, beta=0.0, limit=0.0,
                              fusion="stacked", out_dtype="f32"):
    return _orig_swiglu_op(gate, up, alpha, beta, limit, "stacked", out_dtype)


_orig_permute_align = O.permute_align
_orig_pre_permute = O.pre_permute
_orig_gemm_layout = O.grouped_gemm_layout
_orig_combine = O.combine


def _align_extra_block(topk_ids, num_experts, block_size):
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    numel, E, bs = ids.size, num_experts, block_size
    length = numel + (E + 1) * (bs - 1)
    st = np.full(length, numel, dtype=np.int64)
    blk = np.full(-(-length // bs), -1, dtype=np.int64)
    start = 0
    for e in range(E):
        routes = np.nonzero(ids == e)[0]
        padded = (routes.size // bs) * bs + (bs if routes.size else 0)  # one block too many
        st[start:start + routes.size] = routes
        blk[start // bs:(start + padded) // bs] = e
        start += padded
    return st, blk, start


def _pre_permute_keeps_last(hidden, topk_ids, num_experts, layout, block_size=1, max_m=None):
    if layout != "masked":
        return _orig_pre_permute(hidden, topk_ids, num_experts, layout, block_size, max_m)
    x = np.asarray(hidden, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    K = np.asarray(topk_ids).shape[-1]
    E, H = num_experts, x.shape[1]
    inv = np.full(ids.size, -1, dtype=np.int64)
    out = np.full((E, max_m, H), np.nan)
    cnt = np.zeros(E, dtype=np.int64)
    for e in range(E):
        rt = np.nonzero(ids == e)[0][-max_m:]
        cnt[e] = rt.size
        out[e, :rt.size] = x[rt // K]
        inv[rt] = e * max_m + np.arange(rt.size)
    return out, cnt, inv


def _gemm_layout_per_row_shifted(a, b, layout, metadata, bias=None, act=None, out_dtype="f32"):
    if layout == "per_row":
        metadata = np.where(np.asarray(metadata) >= 0, (np.asarray(metadata) + 1) % len(b), -1)
    return _orig_gemm_layout(a, b, layout, metadata, bias, act, out_dtype)


def _combine_no_skip(y, topk_weights, route_pos, scale=1.0, out_dtype="f32"):
    w = np.asarray(topk_weights, dtype=np.float64)
    T, K = w.shape
    yy = np.asarray(y, dtype=np.float64).reshape(-1, np.asarray(y).shape[-1])
    pos = np.asarray(route_pos, dtype=np.int64).reshape(T, K)
    out = np.zeros((T, yy.shape[1]))
    for k in range(K):
        out += w[:, k:k + 1] * yy[pos[:, k]]
    return O.round_to(float(scale) * out, out_dtype)


MUTANTS = {
    "permute_align pads an exact multiple by one more block": ("permute_align", _align_extra_block),
    "masked slab keeps the last routes": ("pre_permute", _pre_permute_keeps_last),
    "per_row layout reads the next expert": ("grouped_gemm_layout", _gemm_layout_per_row_shifted),
    "combine reads row -1 for a dropped route": ("combine", _combine_no_skip),
    "gelu by its tanh approximation": ("gelu", _gelu_tanh),
    "gelu_and_mul activates the up half": ("gated", _gated_act_on_up),
    "swiglu op reads interleaved input as stacked": ("swiglu_op", _swiglu_op_ignores_fusion),
    "fp8 decoded with bias 8": ("decode_e4m3fn", _decode_fnuz),
    "fp8 b scale tiled along n": ("grouped_gemm_fp8_masked", _fp8_block_scale_tiled),
    "fp8 negative count read as its magnitude": ("grouped_gemm_fp8_masked",
                                                 _fp8_counts_unclamped),
    "fp8 a scale dropped": ("grouped_gemm_fp8_masked", _fp8_no_a_scale),
    "gate clamped from below too": ("swiglu", _swiglu_two_sided_gate),
    "limit<=0 does not disable the clamp": ("swiglu", _swiglu_no_disable),
    "gate and up halves swapped": ("split_gate_up", _split_swapped),
    "ties go to the higher index": ("ranked", _ranked_high_index),
    "scaling factor applied twice": ("routing_weights", _weights_rsf_twice),
    "renormalized over all experts": ("routing_weights", _weights_biased),
    "combine reads route_pos transposed": ("combine", _combine_transposed),
    "down bias dropped": ("expert_mlp", _expert_mlp_no_down_bias),
    "activation not stored in the operand dtype": ("expert_mlp", _expert_mlp_unrounded_act),
    "rounding truncates": ("round_to", _round_truncate),
    "sqrt_softplus drops a term": ("scores", _scores_sqrt_softplus_wrong),
    "biased group score is the max": ("select_experts", _group_max_with_bias),
    "permute not stable": ("permute", _permute_unstable),
    "no-local-expert scale not zero": ("ep_router_outputs", _ep_fill_everywhere_zero_scale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake: {name}"
