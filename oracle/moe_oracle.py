"""Plain, slow, float64 CPU oracle of the routed Mixture-of-Experts FFN forward.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only callers. The GPU library neither imports nor links
anything here, and nothing here comes from the GPU library.

Every function below is the plain definition of one step, written from these pages
(cited by title and section):

  [MR]   ONNX Runtime pull request 32126, "[CUDA] Add MoERouter and SwiGLU contrib
         operators" (sections MoERouter, SwiGLU).
  [CPU]  onnx-light-cpu, "MoE (CPU)" kernel schema (Inputs, Attributes).
  [SPEC] ONNX Runtime pull request 25619, "Update MoE and qMoE spec" (SwiGLU
         Activation Function, Fusion Behavior).
  [TO]   TileOPs, "MoE Operators" API page (one section per op).

Arithmetic is float64. Values are rounded to a storage format (f32, bf16, f16) only
where the pages put a rounding: selection compares float32 scores, the gated
activation is stored in the operand dtype before the down projection, and the outputs
are stored in their dtypes. Matrix products use numpy's float64 matmul as a library
step; there is no tiling, fusion or reordering beyond the definitions.

Where the pages leave a point open, the reading taken is stated at the function.
Parity status of each function is listed in PARITY_STATUS at the end of this file.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "FORMATS", "round_to", "sigmoid", "scores", "ranked", "selection_keys", "select_experts",
    "routing_weights", "ep_router_outputs", "RouteResult", "route", "swiglu", "gelu",
    "gated", "swiglu_op", "ACTIVATIONS", "split_gate_up", "expert_mlp", "grouped_gemm",
    "grouped_gemm_act",
    "permute", "combine", "permute_align", "pre_permute", "grouped_gemm_layout",
    "shared_expert_mlp", "moe_ffn_forward",
    "indexed_backend_applies", "decode_e4m3fn", "grouped_gemm_fp8_masked", "PARITY_STATUS",
]

# --------------------------------------------------------------------------------------
# Storage formats. (significant bits incl. the implicit one, min normal exponent,
# max exponent). bf16 keeps float32's exponent range with 8 significant bits.
FORMATS = {
    "f32": (24, -126, 127),
    "bf16": (8, -126, 127),
    "f16": (11, -14, 15),
}


def round_to(x, fmt: str) -> np.ndarray:
    """Round to the nearest value representable in `fmt`, ties to even; float64 out.

    Direct from float64 (no intermediate rounding): the value is scaled by the power of
    two that makes the format's last kept bit the units digit, rounded to an integer
    with ties to even, and scaled back. Both scalings are exact. Subnormals use the
    fixed spacing of the format's smallest normal binade; magnitudes that round above
    the largest finite value become infinities, as IEEE 754 round-to-nearest does.
    """
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f64":
        return x.copy()
    p, emin, emax = FORMATS[fmt]
    out = np.array(x, dtype=np.float64, copy=True)
    m = np.isfinite(x) & (x != 0.0)
    xf = x[m]
    _, e = np.frexp(xf)  # xf = f * 2**e with 0.5 <= |f| < 1
    ulp_exp = np.maximum(e - p, emin - p + 1)
    r = np.ldexp(np.rint(np.ldexp(xf, -ulp_exp)), ulp_exp)
    maxval = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax
    r = np.where(np.abs(r) > maxval, np.copysign(np.inf, r), r)
    out[m] = r
    return out


def sigmoid(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------------------
# Router: scoring.  [MR] MoERouter (scoring attribute: sqrt_softplus | softmax | sigmoid);
# [TO] FusedTopKFwdOp (scoring runs in float32 whatever the logits dtype).
def scores(logits, scoring: str) -> np.ndarray:
    """Affinity of every expert for every token, float64, over ALL E experts.

    softmax: exp(z_e) / sum_j exp(z_j) (shifted by the row max, which cancels).
    sigmoid: 1 / (1 + exp(-z)).
    sqrt_softplus: the pages only name it; reading taken: sqrt(softplus(z)) with
    softplus(z) = log(1 + exp(z)), written as max(z,0) + log1p(exp(-|z|)).
    The softmax runs over all experts even for an expert-parallel slice: [MR] builds the
    slice's router row so that the result is the globally correct weight.
    """
    z = np.asarray(logits, dtype=np.float64)
    if scoring == "softmax":
        ez = np.exp(z - z.max(axis=-1, keepdims=True))
        return ez / ez.sum(axis=-1, keepdims=True)
    if scoring == "sigmoid":
        return sigmoid(z)
    if scoring == "sqrt_softplus":
        return np.sqrt(np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z))))
    raise ValueError(f"unknown scoring {scoring!r}")


def ranked(values) -> np.ndarray:
    """Indices ordered by value descending, equal values by index ascending.

    [MR] MoERouter: ties go to the lower expert index; [TO] FusedTopKFwdOp: group ties go
    to the lower group index. -0.0 and +0.0 compare equal here.
    """
    v = np.asarray(values, dtype=np.float64)
    return np.lexsort((np.arange(v.size), -v))


def selection_keys(s, correction_bias=None, num_expert_group: int = 1):
    """The float32 selection keys and group scores the top-k compares.

    [MR] MoERouter (noaux_tc adds the bias to the scores before the top-k); [TO]
    FusedMoEFwdOp and FusedTopKFwdOp (DeepSeek-V3 grouped routing).

    u_e = f32(s_e), or f32(f32(s_e) + f32(bias_e)) with a bias. With G groups of E/G
    consecutive experts, a group's score is f32(largest u + second largest u) when a bias
    is given (a group of one expert: its single u), and its largest score otherwise.
    Returns (u [T,E], gs [T,G]); gs is None without groups.
    """
    s32 = round_to(s, "f32")
    T, E = s32.shape
    if correction_bias is None:
        u = s32
    else:
        u = round_to(s32 + round_to(np.asarray(correction_bias, np.float64), "f32")[None, :],
                     "f32")
    G = int(num_expert_group)
    if G <= 1:
        return u, None
    ug = u.reshape(T, G, E // G)
    if correction_bias is not None and E // G >= 2:
        top2 = np.sort(ug, axis=2)[:, :, -2:]
        gs = round_to(top2[:, :, 1] + top2[:, :, 0], "f32")
    elif correction_bias is not None:
        gs = ug[:, :, 0].copy()
    else:
        gs = ug.max(axis=2)
    return u, gs


def select_experts(s, top_k: int, correction_bias=None, num_expert_group: int = 1,
                   topk_group: int = 1):
    """Top-k selection in float32, with optional bias and group limit.

    [MR] MoERouter (selection topk | noaux_tc); [TO] FusedMoEFwdOp and FusedTopKFwdOp.
    The keys and group scores are those of selection_keys(); the topk_group best groups
    (ties to the lower group) stay eligible, and the K eligible experts with the largest
    key are returned in (key descending, index ascending) order.

    Also returns the near-tie diagnostics: gap_sel[t], the smallest difference between
    consecutive keys among the K+1 best eligible experts (it covers the kept/dropped
    boundary and the order inside the row), and gap_group[t], the difference between
    the last kept and the first dropped group score (inf without groups).
    """
    u, gs_all = selection_keys(s, correction_bias, num_expert_group)
    T, E = u.shape
    G, TG, K = int(num_expert_group), int(topk_group), int(top_k)
    group_of = np.arange(E) // (E // G)
    sel = np.zeros((T, K), dtype=np.int64)
    gap_sel = np.full(T, np.inf)
    gap_group = np.full(T, np.inf)
    for t in range(T):
        eligible = np.ones(E, dtype=bool)
        if G > 1:
            gs = gs_all[t]
            gorder = ranked(gs)
            eligible = np.isin(group_of, gorder[:TG])
            if TG < G:
                gap_group[t] = gs[gorder[TG - 1]] - gs[gorder[TG]]
        cand = np.nonzero(eligible)[0]
        order = cand[ranked(u[t, cand])]
        sel[t] = order[:K]
        top = u[t, order[:K + 1]]
        if top.size >= 2:
            gap_sel[t] = np.min(top[:-1] - top[1:])
    return sel, gap_sel, gap_group


def routing_weights(s, sel, renormalize: bool, routed_scaling_factor: float):
    """Weights of the chosen experts.

    [MR]: the weights are the chosen experts' affinities, normalized to sum to one.
    [TO] FusedTopKFwdOp: the returned weights are the unbiased scores of the selected
    experts, renormalized when asked, then multiplied by routed_scaling_factor (applied
    once, after renormalization). Returns (wn, w): wn before the scaling factor.
    Reading: no epsilon in the denominator (the pages give none).
    """
    w = np.take_along_axis(np.asarray(s, np.float64), np.asarray(sel), axis=1)
    wn = w / w.sum(axis=1, keepdims=True) if renormalize else w
    return wn, wn * float(routed_scaling_factor)


def ep_router_outputs(sel, wn, routed_scaling_factor: float, local_expert_start: int,
                      local_expert_count: int, dtype: str):
    """The expert-parallel router row and scale of [MR] MoERouter.

    router_probs[t, j] (expert local_expert_start + j) holds log(wn) for a chosen local
    expert and a large negative fill elsewhere: -1e30, or -1e4 for float16, which cannot
    hold -1e30. A softmax over that row gives wn_e / W_local, W_local being the sum of wn
    over the chosen local experts. weight_scale[t] = route_scale * W_local, exactly zero
    when no chosen expert is local. Readings: route_scale is routed_scaling_factor; the
    logged weight is wn (before the scaling factor); both outputs are stored in `dtype`.
    """
    fill = -1.0e4 if dtype == "f16" else -1.0e30
    sel = np.asarray(sel)
    T, K = sel.shape
    rp = np.full((T, local_expert_count), fill, dtype=np.float64)
    w_local = np.zeros(T, dtype=np.float64)
    for t in range(T):
        for k in range(K):
            e = int(sel[t, k])
            if local_expert_start <= e < local_expert_start + local_expert_count:
                rp[t, e - local_expert_start] = math.log(wn[t, k])
                w_local[t] += wn[t, k]
    return round_to(rp, dtype), round_to(float(routed_scaling_factor) * w_local, dtype)


@dataclass
class RouteResult:
    scores: np.ndarray        # [T,E] float64 affinities
    topk_ids: np.ndarray      # [T,K] int64
    wn: np.ndarray            # [T,K] float64 weights before routed_scaling_factor
    topk_weights: np.ndarray  # [T,K] float32 values (held in float64)
    gap_sel: np.ndarray       # [T] near-tie diagnostic (inf for hash routing)
    gap_group: np.ndarray     # [T]
    router_probs: Optional[np.ndarray] = None
    weight_scale: Optional[np.ndarray] = None
    keys: Optional[np.ndarray] = None          # [T,E] float32 selection keys (diagnostic)
    group_scores: Optional[np.ndarray] = None  # [T,G] group scores, None without groups


def route(logits, top_k: int, scoring: str = "softmax", renormalize: bool = False,
          routed_scaling_factor: float = 1.0, num_expert_group: int = 1,
          topk_group: int = 1, correction_bias=None, expert_ids=None,
          local_expert_start: int = 0, local_expert_count: Optional[int] = None,
          router_probs_dtype: Optional[str] = None) -> RouteResult:
    """The whole router: scores, selection (or hash override), weights, EP outputs.

    [MR]: a given expert_ids replaces the selection for that token (hash routing) and
    the bias is then ignored; the weights still come from the scores of those experts.
    router_probs / weight_scale are produced when router_probs_dtype is given.
    """
    s = scores(logits, scoring)
    T = s.shape[0]
    if expert_ids is not None:
        sel = np.asarray(expert_ids, dtype=np.int64).reshape(T, top_k)
        gap_sel = np.full(T, np.inf)
        gap_group = np.full(T, np.inf)
    else:
        sel, gap_sel, gap_group = select_experts(s, top_k, correction_bias,
                                                 num_expert_group, topk_group)
    wn, w = routing_weights(s, sel, renormalize, routed_scaling_factor)
    res = RouteResult(s, sel, wn, round_to(w, "f32"), gap_sel, gap_group)
    res.keys, res.group_scores = selection_keys(s, correction_bias, num_expert_group)
    if router_probs_dtype is not None:
        count = s.shape[1] - local_expert_start if local_expert_count is None \
            else local_expert_count
        res.router_probs, res.weight_scale = ep_router_outputs(
            sel, wn, routed_scaling_factor, local_expert_start, count, router_probs_dtype)
    return res


# --------------------------------------------------------------------------------------
# Gated activation.  [MR] SwiGLU; [SPEC] SwiGLU Activation Function; [TO]
# MoEGroupedGemmFwdOp (silu_and_mul, swigluoai); [CPU] Attributes (alpha 1, beta 0).
def swiglu(g, l, alpha: float = 1.0, beta: float = 0.0, limit: float = 0.0) -> np.ndarray:
    """G * sigmoid(alpha * G) * (L + beta), G = min(g, limit), L = clamp(l, -limit, limit).

    The gate is clamped from above only, the linear half from both sides, and a limit
    of zero or less turns both clamps off.
    """
    g = np.asarray(g, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    if limit > 0.0:
        g = np.minimum(g, limit)
        l = np.clip(l, -limit, limit)
    return g * sigmoid(alpha * g) * (l + beta)


def gelu(x) -> np.ndarray:
    """x * Phi(x), Phi the standard normal distribution function, = x (1 + erf(x/sqrt 2))/2.

    [TO] MoEGroupedGemmFwdOp names gelu_and_mul = act(gate) * up without fixing the GELU
    form; the reading taken is the exact one (Hendrycks and Gimpel's definition), not the
    tanh approximation.
    """
    x = np.asarray(x, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


# name -> (row layout of gate_up, alpha, beta, limit, kind).  [TO] MoEGroupedGemmFwdOp:
# silu_and_mul and gelu_and_mul read gate rows then up rows and keep act(gate) * up;
# swigluoai reads interleaved rows (2j gate, 2j+1 up) with fixed constants 1.702, 1, 7.
ACTIVATIONS = {
    "silu_and_mul": ("stacked", 1.0, 0.0, 0.0, "swiglu"),
    "swigluoai": ("interleaved", 1.702, 1.0, 7.0, "swiglu"),
    "gelu_and_mul": ("stacked", 0.0, 0.0, 0.0, "gelu"),
}


def gated(g, l, params) -> np.ndarray:
    """The gated activation of a (layout, alpha, beta, limit, kind) tuple on gate g and up l:
    swiglu(g, l, alpha, beta, limit), or gelu(g) * l."""
    _, alpha, beta, limit, kind = params
    if kind == "gelu":
        return gelu(g) * np.asarray(l, dtype=np.float64)
    return swiglu(g, l, alpha, beta, limit)


def swiglu_op(gate, up=None, alpha: float = 1.0, beta: float = 0.0, limit: float = 0.0,
              fusion: str = "stacked", out_dtype: str = "f32") -> np.ndarray:
    """[MR] SwiGLU operator: swiglu of gate and up, float arithmetic, stored in out_dtype.

    With up given, gate and up are [.., F]. Without it gate is [.., 2F] holding both halves
    of one projection: gate first, then up ([MR], fusion "stacked" = [SPEC] swiglu_fusion 2)
    or interleaved per element pair ([SPEC] swiglu_fusion 1).
    """
    if up is None:
        gate, up = split_gate_up(gate, fusion)
    return round_to(swiglu(gate, up, alpha, beta, limit), out_dtype)


def split_gate_up(h, layout: str):
    """Split a [.., 2F] gate/up product. stacked: [gate | up]; interleaved: 2j gate, 2j+1 up.

    [SPEC] Fusion Behavior (fusion 2 concatenated, fusion 1 interleaved); [TO]
    MoEGroupedGemmFwdOp.
    """
    h = np.asarray(h)
    F = h.shape[-1] // 2
    if layout == "stacked":
        return h[..., :F], h[..., F:]
    if layout == "interleaved":
        return h[..., 0::2], h[..., 1::2]
    raise ValueError(f"unknown layout {layout!r}")


def _act_params(act):
    if isinstance(act, str):
        return ACTIVATIONS[act]
    act = tuple(act)  # (layout, alpha, beta, limit[, kind])
    return act if len(act) == 5 else act + ("swiglu",)


def expert_mlp(x, w_gate_up, w_down, b_gate_up=None, b_down=None,
               act="silu_and_mul", act_dtype: str = "f32"):
    """One expert applied to rows x: returns (a, y).

    [TO] MoEExpertMLPFwdOp / MoEGroupedGemmFwdOp: h = x W_gu^T + b_gu (bias added to the
    float product before the activation), a = act(h) stored in the operand dtype, and
    y = a W_d^T + b_d. w_gate_up is [2F, H] and w_down [H, F], each row contiguous
    ([CPU] expert-major, output-major; [SPEC] column-major [H, 2F] storage is the same
    bytes). y is returned unrounded.
    """
    params = _act_params(act)
    layout = params[0]
    x = np.asarray(x, dtype=np.float64)
    h = x @ np.asarray(w_gate_up, dtype=np.float64).T
    if b_gate_up is not None:
        h = h + np.asarray(b_gate_up, dtype=np.float64)[None, :]
    g, l = split_gate_up(h, layout)
    a = round_to(gated(g, l, params), act_dtype)
    y = a @ np.asarray(w_down, dtype=np.float64).T
    if b_down is not None:
        y = y + np.asarray(b_down, dtype=np.float64)[None, :]
    return a, y


# --------------------------------------------------------------------------------------
# Stages on the expert-contiguous (tight) layout.  [TO] MoEGroupedGemmFwdOp (contiguous
# layout: each expert owns one run of consecutive rows), MoEPermuteAlignFwdOp,
# MoEPostPermuteFwdOp.
def grouped_gemm(a, b, expert_offsets, bias=None, out_dtype: str = "f32") -> np.ndarray:
    """out[rows of e] = a[rows of e] @ b[e]^T (+ bias[e]); rows of e are
    expert_offsets[e] .. expert_offsets[e+1]-1. Rows outside every segment stay zero."""
    a = np.asarray(a, dtype=np.float64)
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = off.size - 1
    N = np.asarray(b[0]).shape[0]
    out = np.zeros((a.shape[0], N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            out[lo:hi] = a[lo:hi] @ np.asarray(b[e], dtype=np.float64).T
            if bias is not None:
                out[lo:hi] += np.asarray(bias[e], dtype=np.float64)[None, :]
    return round_to(out, out_dtype)


def grouped_gemm_act(a, b, expert_offsets, act="silu_and_mul", bias=None,
                     out_dtype: str = "f32") -> np.ndarray:
    """The grouped GEMM with the gated activation applied to its float product.

    [TO] MoEGroupedGemmFwdOp with activation: b is [E, 2F, K] in the activation's row
    order, the optional bias is [E, 2F] in the same order and joins before the
    activation; the output has F columns in out_dtype.
    """
    params = _act_params(act)
    h = grouped_gemm(a, b, expert_offsets, bias, "f64")
    g, l = split_gate_up(h, params[0])
    return round_to(gated(g, l, params), out_dtype)


def permute(topk_ids, num_experts: int):
    """Expert-contiguous order of the T*K routes (route r = t*K + k).

    counts[e] routes on expert e; expert_offsets = exclusive prefix sum (E+1 entries);
    sorted_route lists the routes of expert 0, then expert 1, ...; route_pos is its
    inverse. [TO] MoEPermuteAlignFwdOp leaves the order inside an expert's run open;
    the order fixed here is ascending route index.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(ids, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_route = np.argsort(ids, kind="stable")
    route_pos = np.empty_like(sorted_route)
    route_pos[sorted_route] = np.arange(ids.size)
    return offsets, sorted_route, route_pos


def combine(y, topk_weights, route_pos, scale: float = 1.0, out_dtype: str = "f32"):
    """out[t] = scale * sum_k topk_weights[t,k] * y[route_pos[t*K + k]], k ascending.

    [TO] MoEPostPermuteFwdOp: back to token order, routing weights applied, top-k
    reduced, then the cast. Works for every layout: route_pos is the layout's inverse
    index (the row of y holding route t*K + k). A negative position (a route a masked
    slab had no room for) contributes nothing; the pages leave capacity overflow open and
    this is the reading taken.
    """
    w = np.asarray(topk_weights, dtype=np.float64)
    T, K = w.shape
    y = np.asarray(y, dtype=np.float64).reshape(-1, np.asarray(y).shape[-1])
    pos = np.asarray(route_pos, dtype=np.int64).reshape(T, K)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for k in range(K):
        live = pos[:, k] >= 0
        out[live] += w[live, k:k + 1] * y[pos[live, k]]
    return round_to(float(scale) * out, out_dtype)


# --------------------------------------------------------------------------------------
# Padded and masked layouts.  [TO] MoEPermuteAlignFwdOp, MoEPrePermuteFwdOp,
# MoEGroupedGemmFwdOp (layout table: contiguous with segment ends, contiguous with a
# per-row expert id, masked [E, max_m, K] with valid counts), MoEPostPermuteFwdOp.
def permute_align(topk_ids, num_experts: int, block_size: int):
    """[TO] MoEPermuteAlignFwdOp: routes grouped by expert, each expert's range padded up
    to a multiple of block_size.

    Returns (sorted_token_ids, expert_ids, num_tokens_post_pad) with numel = T*K routes:
    sorted_token_ids has numel + (E+1)(block_size-1) entries; expert e's range holds its
    routes (ascending route index: the pages leave the order open) followed by numel up
    to the padded length; every entry past num_tokens_post_pad is numel. expert_ids has
    ceil(len / block_size) entries: the owner of each block of the ranges, then -1 (a
    value outside [0, E)).
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    numel, E, bs = ids.size, num_experts, block_size
    length = numel + (E + 1) * (bs - 1)
    sorted_ids = np.full(length, numel, dtype=np.int64)
    blocks = np.full(-(-length // bs), -1, dtype=np.int64)
    start = 0
    for e in range(E):
        routes = np.nonzero(ids == e)[0]
        padded = -(-routes.size // bs) * bs
        sorted_ids[start:start + routes.size] = routes
        blocks[start // bs:(start + padded) // bs] = e
        start += padded
    return sorted_ids, blocks, start


def pre_permute(hidden, topk_ids, num_experts: int, layout: str, block_size: int = 1,
                max_m: Optional[int] = None):
    """[TO] MoEPrePermuteFwdOp: (expert_input, layout_metadata, inverse_indices).

    layout "contiguous" (segment ends) or "per_row" (expert id per row): the rows of
    permute_align(..., block_size) (block_size 1 = the tight layout), expert_input
    [numel + E (block_size - 1), H] with pad rows and rows past the used length NaN
    (unspecified); metadata = the E segment ends, or the expert of each row (-1 on pad
    and unused rows). layout "masked": expert_input [E, max_m, H], metadata = rows placed
    per expert, min(count, max_m); a route ranked max_m or later in its expert has no
    room (inverse -1, the reading taken where the pages are silent). inverse_indices [T*K]:
    the row of expert_input (flattened) holding route r = t*K + k, which reads hidden[t].
    """
    x = np.asarray(hidden, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    K = np.asarray(topk_ids).shape[-1]
    numel, E, H = ids.size, num_experts, x.shape[1]
    inverse = np.full(numel, -1, dtype=np.int64)
    if layout == "masked":
        out = np.full((E, max_m, H), np.nan)
        counts = np.zeros(E, dtype=np.int64)
        for e in range(E):
            routes = np.nonzero(ids == e)[0][:max_m]
            counts[e] = routes.size
            out[e, :routes.size] = x[routes // K]
            inverse[routes] = e * max_m + np.arange(routes.size)
        return out, counts, inverse
    sorted_ids, blocks, used = permute_align(ids, E, block_size)
    cap = numel + E * (block_size - 1)
    out = np.full((cap, H), np.nan)
    live = np.nonzero(sorted_ids[:used] < numel)[0]
    out[live] = x[sorted_ids[live] // K]
    inverse[sorted_ids[live]] = live
    if layout == "per_row":
        meta = np.full(cap, -1, dtype=np.int64)
        meta[live] = ids[sorted_ids[live]]
        return out, meta, inverse
    if layout == "contiguous":
        ends = np.zeros(E, dtype=np.int64)
        for e in range(E):
            own = np.nonzero(blocks == e)[0]
            ends[e] = (own[-1] + 1) * block_size if own.size else (ends[e - 1] if e else 0)
        return out, ends, inverse
    raise ValueError(f"unknown layout {layout!r}")


def grouped_gemm_layout(a, b, layout: str, metadata, bias=None, act=None,
                        out_dtype: str = "f32") -> np.ndarray:
    """[TO] MoEGroupedGemmFwdOp over one of its layouts: out[rows of g] = a[rows of g]
    b[g]^T (+ bias[g]), then the gated activation when act is given (F = N/2 columns).

    contiguous: a [M, K], metadata = E segment ends (expert g owns rows end[g-1] ..
    end[g]-1, end[-1] = 0). per_row: a [M, K], metadata [M] = expert of each row (rows
    whose id is outside [0, E) belong to none). masked: a [E, max_m, K], metadata [E] =
    valid rows, read as max_m when larger and 0 when negative. Rows owned by no expert,
    and masked rows past the count, are NaN (unspecified).
    """
    b = [np.asarray(b[g], dtype=np.float64) for g in range(len(b))]
    E, N = len(b), b[0].shape[0]
    meta = np.asarray(metadata, dtype=np.int64)
    a = np.asarray(a, dtype=np.float64)
    masked = layout == "masked"
    rows = a.reshape(-1, a.shape[-1])
    owner = np.full(rows.shape[0], -1, dtype=np.int64)
    if masked:
        max_m = a.shape[1]
        for g in range(E):
            c = int(min(max(meta[g], 0), max_m))
            owner[g * max_m:g * max_m + c] = g
    elif layout == "contiguous":
        lo = 0
        for g in range(E):
            owner[lo:meta[g]] = g
            lo = meta[g]
    elif layout == "per_row":
        ok = (meta >= 0) & (meta < E)
        owner[ok] = meta[ok]
    else:
        raise ValueError(f"unknown layout {layout!r}")
    h = np.full((rows.shape[0], N), np.nan)
    for m in np.nonzero(owner >= 0)[0]:
        g = owner[m]
        h[m] = b[g] @ rows[m]
        if bias is not None:
            h[m] += np.asarray(bias[g], dtype=np.float64)
    if act is not None:
        params = _act_params(act)
        gg, l = split_gate_up(h, params[0])
        h = gated(gg, l, params)
    out = round_to(h, out_dtype)
    return out.reshape(*a.shape[:-1], out.shape[-1])


def shared_expert_mlp(x, w_gate_up, w_down, dtype: str) -> np.ndarray:
    """[TO] SharedExpertMLPFwdOp: down(silu(x G^T) * (x U^T)).

    w_gate_up is [2S, H], the S gate rows then the S up rows; w_down is [H, S]. The
    gated activation is stored in the input dtype before the down projection; the
    result is stored in the input dtype.
    """
    x = np.asarray(x, dtype=np.float64)
    wgu = np.asarray(w_gate_up, dtype=np.float64)
    S = wgu.shape[0] // 2
    h = x @ wgu.T
    a = round_to(h[:, :S] * sigmoid(h[:, :S]) * h[:, S:], dtype)
    return round_to(a @ np.asarray(w_down, dtype=np.float64).T, dtype)


def moe_ffn_forward(hidden, logits, w_gate_up, w_down, *, top_k: int,
                    scoring: str = "softmax", renormalize: bool = False,
                    routed_scaling_factor: float = 1.0, num_expert_group: int = 1,
                    topk_group: int = 1, act="silu_and_mul", dtype: str = "bf16",
                    correction_bias=None, expert_ids=None, b_gate_up=None, b_down=None,
                    shared_w_gate_up=None, shared_w_down=None, tokens=None):
    """Routed MoE FFN forward (plus the optional shared expert) for the given tokens.

    [TO] FusedMoEFwdOp / FusedMoEExpertsFwdOp / FusedMoESharedExpertFwdOp:
      out[t] = sum_k w[t,k] * (down_k(act(gate_up_k(h_t) + b_gu)) + b_down)
    where w already holds routed_scaling_factor (applied once), stored in `dtype`;
    shared_out[t] = shared expert of h_t (no scaling factor), returned separately.

    w_gate_up[e] / w_down[e] / b_gate_up[e] / b_down[e] are read one expert at a time
    (any indexable works, so a caller can fetch experts lazily). `tokens` restricts the
    computation to those rows; every step is per token, so the result for a token does
    not depend on which others are computed.
    """
    hidden = np.asarray(hidden)
    tokens = np.arange(hidden.shape[0]) if tokens is None else np.asarray(tokens)
    x = np.asarray(hidden[tokens], dtype=np.float64)
    ids_in = None if expert_ids is None else np.asarray(expert_ids)[tokens]
    r = route(np.asarray(logits)[tokens], top_k, scoring, renormalize,
              routed_scaling_factor, num_expert_group, topk_group, correction_bias, ids_in)
    n, K = r.topk_ids.shape
    y = np.zeros((n, K, x.shape[1]), dtype=np.float64)
    for e in np.unique(r.topk_ids):
        tt, kk = np.nonzero(r.topk_ids == e)
        _, ye = expert_mlp(x[tt], w_gate_up[e], w_down[e],
                           None if b_gate_up is None else b_gate_up[e],
                           None if b_down is None else b_down[e], act, dtype)
        y[tt, kk] = ye
    acc = np.zeros((n, x.shape[1]), dtype=np.float64)
    for k in range(K):
        acc += r.topk_weights[:, k:k + 1] * y[:, k]
    result = {"out": round_to(acc, dtype), "route": r, "tokens": tokens}
    if shared_w_gate_up is not None:
        result["shared_out"] = shared_expert_mlp(x, shared_w_gate_up, shared_w_down, dtype)
    return result


def indexed_backend_applies(T: int, K: int, E: int, H: int, F: int, activation: str,
                            has_bias: bool) -> bool:
    """[TO] FusedMoEExpertsFwdOp: the indexed small-route backend serves a call when
    T*K <= 2E, the activation is silu_and_mul, there is no bias, H % 128 == 0 and
    F % 256 == 0; every other call takes the staged pipeline."""
    return (T * K <= 2 * E and activation == "silu_and_mul" and not has_bias
            and H % 128 == 0 and F % 256 == 0)


# --------------------------------------------------------------------------------------
# Block-scaled FP8 grouped GEMM over a masked slab.

def decode_e4m3fn(codes) -> np.ndarray:
    """float8_e4m3fn codes (bytes) to float64 values.

    [TO] MoEGroupedGemmFP8FwdOp types both operands float8_e4m3fn: the E4M3 encoding of
    the OCP 8-bit floating point formats. Bit 7 is the sign, bits 6..3 the exponent with
    bias 7, bits 2..0 the mantissa. Exponent field 0 holds the subnormals m/8 * 2^-6.
    There are no infinities: only the all-ones exponent with all-ones mantissa is NaN,
    so exponent 15 with mantissa 0..6 are ordinary values up to 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def grouped_gemm_fp8_masked(a_codes, a_scale, b_codes, b_scale, counts) -> np.ndarray:
    """[TO] MoEGroupedGemmFP8FwdOp: one block-scaled FP8 GEMM per expert over a masked slab.

    a [E, max_m, K] and b [E, N, K] are float8_e4m3fn codes; a_scale [E, max_m, K/128]
    holds one float32 per row and 128 columns of a, b_scale [E, N/128, K/128] one per
    128 x 128 block of b; K and N are multiples of 128. Expert g has m_g valid rows,
    counts[g] read as max_m past max_m and as 0 below 0. For each 128-wide K block kb the
    raw FP8 values are contracted, the block sum is multiplied by its two scales
    a_scale[g, m, kb] * b_scale[g, n // 128, kb], and the products are added up:
        out[g, m, n] = sum_kb (sum_{k in kb} a[g,m,k] b[g,n,k]) a_scale[g,m,kb] b_scale[g,n//128,kb]
    stored in bfloat16. Rows at or past m_g are undefined on the page; they are NaN here.
    Sums are float64 (the page's accuracy reference is the dequantized product).
    """
    A = decode_e4m3fn(a_codes)
    B = decode_e4m3fn(b_codes)
    sa = np.asarray(a_scale, dtype=np.float64)
    sb = np.asarray(b_scale, dtype=np.float64)
    E, max_m, K = A.shape
    N = B.shape[1]
    out = np.full((E, max_m, N), np.nan)
    for g in range(E):
        m = int(min(max(int(counts[g]), 0), max_m))
        acc = np.zeros((m, N))
        for kb in range(K // 128):
            ks = slice(128 * kb, 128 * (kb + 1))
            block = A[g, :m, ks] @ B[g, :, ks].T
            acc += block * sa[g, :m, kb][:, None] * np.repeat(sb[g, :, kb], 128)[None, :]
        out[g, :m] = round_to(acc, "bf16")
    return out


# What pins each function (the tests under tests/ named test_oracle_*.py). Functions
# whose parity rests only on a reading of the pages say so.
PARITY_STATUS = {
    "round_to": "pinned: numpy float32/float16 casts, torch bfloat16 cast, brute force",
    "scores": "pinned: decimal-arithmetic closed forms, softmax invariants",
    "select_experts": "pinned: brute-force subset enumeration, constructed ties",
    "routing_weights": "pinned: closed forms (sum to one, softmax of the chosen logits)",
    "ep_router_outputs": "pinned: softmax-of-row invariant, zero-scale rule, rank sum",
    "swiglu": "pinned: decimal-arithmetic closed forms, clamp-disable rule",
    "expert_mlp": "pinned: E=1 dense gated MLP (torch float64), soft mixture",
    "grouped_gemm": "pinned: per-row brute-force dot products",
    "permute": "pinned: permutation invariants, brute-force stable order",
    "combine": "pinned: brute-force per-element sums",
    "shared_expert_mlp": "pinned: torch float64 dense MLP with rounding points",
    "moe_ffn_forward": "pinned: soft-mixture special case, per-token brute force",
    "decode_e4m3fn": "pinned: torch float8_e4m3fn decode of all 256 codes, format constants",
    "grouped_gemm_fp8_masked": "pinned: dequantize-then-multiply brute force, exact small "
                               "integers, count clamping",
    "gelu": "pinned: tabulated normal distribution function (15 decimals), torch's exact "
            "GELU, GELU(x) - GELU(-x) = x",
    "gated": "pinned: gelu_and_mul brute force against torch's GELU; swiglu as above",
    "swiglu_op": "pinned: separate / stacked / interleaved forms agree, decimal closed "
                 "forms, bf16 store against torch's cast",
    "permute_align": "pinned: the page's definition checked as invariants (per-expert "
                     "route sets, padded lengths, numel fill, block owners, tail values)",
    "pre_permute": "pinned: expert_input[inverse[r]] = hidden[r / K], the tight layout "
                   "against permute(), masked counts and drops against brute-force ranks",
    "grouped_gemm_layout": "pinned: per-row brute-force products; the three layouts of one "
                           "routed problem agree route by route",
    "sqrt_softplus reading": "parity unpinned beyond the reading sqrt(softplus(z))",
    "gelu_and_mul reading": "the exact GELU is a reading (the pages name the activation "
                            "only); pinned as that reading",
}
