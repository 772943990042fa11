"""Pins of the CPU oracle to things other than itself.

Each pin_* function raises AssertionError when the oracle disagrees with a closed form,
a brute-force enumeration, an identity the pages fix, or an independent library routine.
They reach the oracle only through the module object `O`, so test_oracle_mutants.py can
plant a mistake in one oracle function and check that some pin catches it.
"""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import torch

import oracle.moe_oracle as O

getcontext().prec = 60
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "page_constants.json")))


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _D(x):
    return Decimal(float(x))


def _dsig(x):
    return 1 / (1 + (-x).exp())


# ------------------------------------------------------------------- rounding
def pin_round_f32_f16():
    r = _rng(1)
    x = np.concatenate([
        r.standard_normal(4000) * 10.0 ** r.integers(-45, 39, 4000),
        r.standard_normal(500) * 1e-41, np.array([3.5e38, 3.4028235e38, 3.4028236e38, -7e45]),
    ])
    assert np.array_equal(O.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))
    y = np.concatenate([r.standard_normal(4000) * 10.0 ** r.integers(-9, 5, 4000),
                        np.array([65504.0, 65519.99, 65520.0, 1e-8, 6e-8, -3e-5])])
    assert np.array_equal(O.round_to(y, "f16"), y.astype(np.float16).astype(np.float64))


def _all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32).astype(np.float64)
    v = v[np.isfinite(v)]
    v = np.unique(v)          # sorted, -0.0 merged with 0.0
    return v


def pin_round_bf16_bruteforce():
    vals = _all_bf16_values()
    mant_odd = {}
    bits = np.arange(1 << 16, dtype=np.uint32)
    fv = (bits << 16).view(np.float32).astype(np.float64)
    for b, v in zip(bits, fv):
        if np.isfinite(v):
            mant_odd[float(v)] = bool(b & 1)
    r = _rng(2)
    x = np.concatenate([r.standard_normal(3000) * 10.0 ** r.integers(-40, 38, 3000),
                        # exact ties between neighbours
                        (vals[1000:1200] + vals[1001:1201]) / 2.0])
    got = O.round_to(x, "bf16")
    for xi, gi in zip(x, got):
        j = np.searchsorted(vals, xi)
        lo, hi = vals[max(j - 1, 0)], vals[min(j, vals.size - 1)]
        dlo, dhi = abs(xi - lo), abs(hi - xi)
        if dlo < dhi:
            want = lo
        elif dhi < dlo:
            want = hi
        else:
            want = hi if not mant_odd[float(hi)] else lo
        assert gi == want, (xi, gi, want)
    # independent library: torch's float32 -> bfloat16 cast (round to nearest even)
    x32 = r.standard_normal(20000).astype(np.float32)
    t = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to(x32.astype(np.float64), "bf16"), t)


# ------------------------------------------------------------------- scoring
def pin_scores_closed_forms():
    zs = [0.0, 1.0, -1.0, 20.0, -20.0, 3.5, -0.75]
    s = O.scores(np.array([zs]), "sqrt_softplus")[0]
    for z, v in zip(zs, s):
        want = (1 + _D(z).exp()).ln().sqrt()
        assert abs(_D(v) - want) <= Decimal("1e-15") * want, (z, v, want)
    assert abs(s[0] - math.sqrt(math.log(2.0))) < 1e-15
    g = O.scores(np.array([zs]), "sigmoid")[0]
    for z, v in zip(zs, g):
        want = _dsig(_D(z))
        assert abs(_D(v) - want) <= Decimal("1e-15") * want, (z, v)
    assert g[0] == 0.5
    r = _rng(3)
    z = r.standard_normal((5, 9)) * 3
    sm = O.scores(z, "softmax")
    for row_z, row_s in zip(z, sm):
        den = sum(_D(v).exp() for v in row_z)
        for v, p in zip(row_z, row_s):
            want = _D(v).exp() / den
            assert abs(_D(p) - want) <= Decimal("1e-14") * want
    assert np.allclose(sm.sum(axis=1), 1.0, atol=1e-15, rtol=0)
    assert np.allclose(O.scores(z + 100.0, "softmax"), sm, atol=0, rtol=1e-13)


# ------------------------------------------------------------------- selection
def _key(u, e):
    return (-u, e)


def _brute_select(u, K, G=1, TG=1, biased=False):
    """Brute force: enumerate every TG-subset of groups and every K-subset of experts; the
    answer is the unique subset whose members all precede every non-member under
    (value descending, index ascending)."""
    E = u.size
    eligible = list(range(E))
    if G > 1:
        gsz = E // G
        gs = []
        for g in range(G):
            mem = u[g * gsz:(g + 1) * gsz]
            if biased and gsz >= 2:
                best = max(O.round_to(mem[i] + mem[j], "f32")
                           for i in range(gsz) for j in range(gsz) if i != j)
            else:
                best = max(mem)
            gs.append(float(best))
        kept = None
        for sub in itertools.combinations(range(G), TG):
            rest = [g for g in range(G) if g not in sub]
            if all(_key(gs[a], a) < _key(gs[b], b) for a in sub for b in rest):
                assert kept is None
                kept = sub
        eligible = [e for e in range(E) if e // gsz in kept]
    chosen = None
    for sub in itertools.combinations(eligible, K):
        rest = [e for e in eligible if e not in sub]
        if all(_key(u[a], a) < _key(u[b], b) for a in sub for b in rest):
            assert chosen is None
            chosen = sub
    return sorted(chosen, key=lambda e: _key(u[e], e))


def pin_select_bruteforce():
    r = _rng(4)
    cases = [(8, 2, 1, 1, False), (8, 3, 1, 1, True), (16, 3, 4, 2, False),
             (16, 3, 4, 2, True), (12, 4, 3, 2, True), (8, 2, 8, 3, True)]
    for E, K, G, TG, biased in cases:
        for trial in range(25):
            logits = _f32(r.standard_normal((1, E)))
            bias = _f32(r.uniform(-0.1, 0.1, E)) if biased else None
            scoring = "sigmoid" if biased else ["softmax", "sigmoid", "sqrt_softplus"][trial % 3]
            s = O.scores(logits, scoring)
            sel, _, _ = O.select_experts(s, K, bias, G, TG)
            u = _f32(s[0]) if bias is None else O.round_to(_f32(s[0]) + bias, "f32")
            assert list(sel[0]) == _brute_select(u, K, G, TG, biased), (E, K, G, TG, trial)


def pin_select_ties():
    # all-equal logits: ids 0..K-1, weights 1/K * rsf
    res = O.route(np.zeros((2, 8)), 3, "softmax", True, 2.5)
    assert res.topk_ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(res.topk_weights, 2.5 / 3, rtol=1e-7)
    # pairwise-equal keys go to the lower index
    z = np.array([[0.1, 0.9, 0.3, 0.9, 0.3, -1.0]])
    assert O.route(z, 3, "sigmoid").topk_ids.tolist() == [[1, 3, 2]]
    # equal group scores: the lower group is kept
    z = np.array([[0.5, 0.2, 0.2, 0.5, 0.0, 0.0]])
    res = O.route(z, 2, "sigmoid", num_expert_group=3, topk_group=1,
                  correction_bias=np.zeros(6))
    assert res.topk_ids.tolist() == [[0, 1]]
    # negative zero equals zero: index decides
    assert list(O.ranked(np.array([-0.0, 0.0, -0.0]))) == [0, 1, 2]


def pin_group_score_rule():
    # with a bias the group score is the sum of the two best biased scores, not the max
    z = np.zeros((1, 8))
    bias = np.array([0.30, 0.0, 0.0, 0.0, 0.20, 0.20, 0.0, 0.0])
    res = O.route(z, 2, "sigmoid", num_expert_group=2, topk_group=1, correction_bias=bias)
    assert res.topk_ids.tolist() == [[4, 5]]          # 0.7+0.7 > 0.8+0.5
    # selection uses biased keys, weights use unbiased scores
    assert np.allclose(res.wn, [[0.5, 0.5]])
    # without a bias the group score is the best score
    z2 = np.array([[2.0, -5, -5, -5, 1.5, 1.4, 1.3, 1.2]])
    assert O.route(z2, 2, "sigmoid", num_expert_group=2,
                   topk_group=1).topk_ids.tolist() == [[0, 1]]


# ------------------------------------------------------------------- weights
def pin_weights_closed_forms():
    r = _rng(5)
    z = _f32(r.standard_normal((6, 10)))
    res = O.route(z, 4, "softmax", True, 1.7)
    assert np.allclose(res.topk_weights.sum(axis=1), 1.7, rtol=1e-6)
    for t in range(6):
        sub = z[t, res.topk_ids[t]]
        want = np.exp(sub) / np.exp(sub).sum()      # softmax over the chosen logits alone
        assert np.allclose(res.wn[t], want, rtol=1e-13)
    res2 = O.route(z, 4, "sigmoid", False, 1.0)
    assert np.allclose(res2.wn, 1 / (1 + np.exp(-np.take_along_axis(z, res2.topk_ids, 1))),
                       rtol=1e-14)
    # hash routing: the given experts, normalized affinities, bias ignored
    ids = np.array([[3, 1], [0, 9], [5, 4], [2, 8], [7, 6], [9, 0]])
    res3 = O.route(z, 2, "sigmoid", True, 1.0, correction_bias=np.full(10, 5.0),
                   expert_ids=ids)
    assert res3.topk_ids.tolist() == ids.tolist()
    sg = 1 / (1 + np.exp(-np.take_along_axis(z, ids, 1)))
    assert np.allclose(res3.wn, sg / sg.sum(axis=1, keepdims=True), rtol=1e-14)


# ------------------------------------------------------------------- EP router outputs
def pin_ep_outputs():
    fills = GOLDEN["router_probs_fill"]
    r = _rng(6)
    z = _f32(r.standard_normal((40, 16)))
    for dt in ("f32", "bf16", "f16"):
        full = O.route(z, 4, "softmax", True, 2.0, router_probs_dtype=dt)
        assert np.allclose(full.weight_scale, 2.0, rtol=2e-3)  # full slice: W_local = 1
        res = O.route(z, 4, "softmax", True, 2.0, local_expert_start=4,
                      local_expert_count=6, router_probs_dtype=dt)
        fill = O.round_to(fills[dt], dt)
        for t in range(40):
            local = [(k, e) for k, e in enumerate(res.topk_ids[t]) if 4 <= e < 10]
            row = res.router_probs[t]
            if not local:
                assert res.weight_scale[t] == 0.0
                assert np.all(row == fill)
                continue
            sm = np.exp(row - row.max())
            sm = sm / sm.sum()
            rec = res.weight_scale[t] * sm                 # what the consumer rebuilds
            want = np.zeros(6)
            for k, e in local:
                want[e - 4] = res.topk_weights[t, k]
            tol = {"f32": 1e-6, "bf16": 2e-2, "f16": 2e-3}[dt]
            assert np.allclose(rec, want, rtol=tol, atol=tol * 1e-2), (dt, t)
            mask = np.ones(6, bool)
            mask[[e - 4 for _, e in local]] = False
            assert np.all(row[mask] == fill)
    assert O.round_to(-1e30, "f16") == -np.inf        # why float16 needs its own fill
    assert O.round_to(fills["f16"], "f16") == -1e4
    # fake multi-rank: scale_r * softmax(row_r), summed over ranks, is the global weight
    res_all = O.route(z, 4, "softmax", True, 2.0)
    total = np.zeros((40, 16))
    for rank in range(4):
        rr = O.route(z, 4, "softmax", True, 2.0, local_expert_start=4 * rank,
                     local_expert_count=4, router_probs_dtype="f32")
        row = rr.router_probs
        sm = np.exp(row - row.max(axis=1, keepdims=True))
        sm = sm / sm.sum(axis=1, keepdims=True)
        total[:, 4 * rank:4 * rank + 4] = rr.weight_scale[:, None] * sm
    want = np.zeros((40, 16))
    np.put_along_axis(want, res_all.topk_ids, res_all.topk_weights, axis=1)
    assert np.allclose(total, want, rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------------- SwiGLU
def _dswiglu(g, l, alpha, beta, limit):
    g, l = _D(g), _D(l)
    if limit > 0:
        g = min(g, _D(limit))
        l = max(min(l, _D(limit)), -_D(limit))
    return g * _dsig(_D(alpha) * g) * (l + _D(beta))


def pin_swiglu_closed_forms():
    oai = GOLDEN["swigluoai"]
    assert O.ACTIVATIONS["swigluoai"] == ("interleaved", oai["alpha"], oai["beta"],
                                          oai["limit"], "swiglu")
    assert O.ACTIVATIONS["silu_and_mul"][0] == GOLDEN["silu_and_mul"]["layout"]
    cases = [((1.0, 1.0), (1.0, 0.0, 0.0), 0.7310585786300049),
             ((-2.0, 3.0), (1.0, 0.0, 0.0), -0.7152175321327052),
             ((10.0, 10.0), (1.702, 1.0, 7.0), 55.99962502642654),
             ((-10.0, -10.0), (1.702, 1.0, 7.0), 2.434776776913187e-06),
             ((0.5, -0.25), (1.702, 1.0, 7.0), 0.2627913274547851),
             ((10.0, 10.0), (1.702, 1.0, 0.0), 109.99999553624258),
             ((10.0, 10.0), (1.702, 1.0, -1.0), 109.99999553624258),
             ((3.0, -9.0), (1.0, 0.5, 7.0), None), ((-3.0, 9.0), (0.7, -0.5, 2.0), None)]
    for (g, l), (a, b, lim), printed in cases:
        got = float(O.swiglu(g, l, a, b, lim))
        want = _dswiglu(g, l, a, b, lim)
        assert abs(_D(got) - want) <= Decimal("1e-15") * abs(want), (g, l, got, want)
        if printed is not None:
            assert abs(got - printed) <= 4e-16 * abs(printed)


def _torch_dense_gated(x, wg, wu, wd, act_round):
    xt = torch.from_numpy(np.asarray(x, np.float64))
    a = torch.nn.functional.silu(xt @ torch.from_numpy(wg).T) * (xt @ torch.from_numpy(wu).T)
    a = act_round(a)
    return (a @ torch.from_numpy(wd).T).numpy()


def pin_expert_mlp_dense_special_case():
    r = _rng(7)
    T, H, F = 9, 24, 10
    x = _f32(r.standard_normal((T, H)))
    wgu = _f32(r.standard_normal((1, 2 * F, H)) * 0.2)
    wd = _f32(r.standard_normal((1, H, F)) * 0.2)
    z = np.zeros((T, 1))
    out = O.moe_ffn_forward(x, z, wgu, wd, top_k=1, renormalize=True, dtype="f32")["out"]
    ref = _torch_dense_gated(x, wgu[0, :F], wgu[0, F:], wd[0],
                             lambda a: a.to(torch.float32).to(torch.float64))
    assert np.allclose(out, ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    sh = O.shared_expert_mlp(x, wgu[0], wd[0], "f32")
    assert np.allclose(sh, ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    shb = O.shared_expert_mlp(x, wgu[0], wd[0], "bf16")
    refb = _torch_dense_gated(x, wgu[0, :F], wgu[0, F:], wd[0],
                              lambda a: a.to(torch.bfloat16).to(torch.float64))
    assert np.allclose(shb, refb, rtol=1e-2, atol=1e-3)


def pin_layout_and_bias_identities():
    r = _rng(8)
    T, H, F = 7, 16, 6
    x = _f32(r.standard_normal((T, H)))
    w_st = _f32(r.standard_normal((2 * F, H)) * 0.3)
    wd = _f32(r.standard_normal((H, F)) * 0.3)
    # stacked -> interleaved row permutation gives the same MLP
    perm = np.empty(2 * F, dtype=np.int64)
    perm[0::2] = np.arange(F)
    perm[1::2] = F + np.arange(F)
    a1, y1 = O.expert_mlp(x, w_st, wd, act=("stacked", 1.3, 0.2, 1.5), act_dtype="f64")
    a2, y2 = O.expert_mlp(x, w_st[perm], wd, act=("interleaved", 1.3, 0.2, 1.5),
                          act_dtype="f64")
    assert np.allclose(a1, a2, rtol=1e-14) and np.allclose(y1, y2, rtol=1e-13)
    # gate rows really are the gate: swapping halves changes the result
    a3, _ = O.expert_mlp(x, np.concatenate([w_st[F:], w_st[:F]]), wd, act_dtype="f64")
    a4, _ = O.expert_mlp(x, w_st, wd, act_dtype="f64")
    g, u = x @ w_st[:F].T, x @ w_st[F:].T
    assert np.allclose(a4, g / (1 + np.exp(-g)) * u, rtol=1e-13)
    assert not np.allclose(a3, a4)
    # a bias equals one more input column holding 1 (augmentation identity)
    bgu = _f32(r.standard_normal(2 * F) * 0.5)
    bd = _f32(r.standard_normal(H) * 0.5)
    xa = np.concatenate([x, np.ones((T, 1))], axis=1)
    wa = np.concatenate([w_st, bgu[:, None]], axis=1)
    a5, y5 = O.expert_mlp(x, w_st, wd, bgu, bd, act="swigluoai", act_dtype="f64")
    a6, y6 = O.expert_mlp(xa, wa, wd, act="swigluoai", act_dtype="f64")
    assert np.allclose(a5, a6, rtol=1e-13)
    assert np.allclose(y5, y6 + bd[None, :], rtol=1e-13)


def pin_activation_rounding_point():
    """The gated activation is stored in the operand dtype before the down projection.
    One-hot tokens make h a weight column exactly, a down weight of 3 I makes y = 3 a
    exactly, and top-1 routing over one expert gives weight 1; so the layer output is
    bf16(3 bf16(act(h))), which differs from bf16(3 act(h)) on this fixture."""
    r = _rng(31)
    n = 16
    x = np.eye(n)
    wgu = torch.from_numpy(r.standard_normal((1, 2 * n, n))).to(torch.bfloat16)
    wgu = wgu.to(torch.float64).numpy()
    wd = (3.0 * np.eye(n))[None]
    out = O.moe_ffn_forward(x, np.zeros((n, 1)), wgu, wd, top_k=1, renormalize=True,
                            dtype="bf16")["out"]
    g, u = wgu[0, :n].T, wgu[0, n:].T             # h[t] = column t of the weight
    act = g / (1.0 + np.exp(-g)) * u

    def bf(v):
        # torch rounds through float32; that equals one rounding unless the float32 value
        # is a bfloat16 midpoint while v itself is not (checked here)
        v = np.asarray(v, np.float64)
        v32 = v.astype(np.float32)
        mid = (v32.view(np.uint32) & 0xFFFF) == 0x8000
        assert not np.any(mid & (v32.astype(np.float64) != v))
        return torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    want = bf(3.0 * bf(act))
    assert not np.array_equal(want, bf(3.0 * act))  # the fixture tells the two apart
    assert np.array_equal(out, want)


# ------------------------------------------------------------------- stages
def pin_grouped_gemm_bruteforce():
    r = _rng(9)
    E, N, K = 3, 5, 7
    off = np.array([0, 4, 4, 9])
    a = r.standard_normal((9, K))
    b = r.standard_normal((E, N, K))
    bias = r.standard_normal((E, N))
    out = O.grouped_gemm(a, b, off, bias, "f64")
    for e in range(E):
        for m in range(off[e], off[e + 1]):
            for n in range(N):
                want = math.fsum(a[m, k] * b[e, n, k] for k in range(K)) + bias[e, n]
                assert abs(out[m, n] - want) < 1e-12
    b2 = r.standard_normal((E, 2 * 3, K))
    act = O.grouped_gemm_act(a, b2, off, "swigluoai", None, "f64")
    for e in range(E):
        for m in range(off[e], off[e + 1]):
            for j in range(3):
                g = math.fsum(a[m, k] * b2[e, 2 * j, k] for k in range(K))
                u = math.fsum(a[m, k] * b2[e, 2 * j + 1, k] for k in range(K))
                want = float(_dswiglu(g, u, 1.702, 1.0, 7.0))
                assert abs(act[m, j] - want) < 1e-12 * max(1.0, abs(want))


def pin_permute_invariants():
    r = _rng(10)
    for T, K, E in [(13, 3, 5), (40, 2, 9), (1, 1, 1), (0, 2, 4)]:
        ids = np.stack([r.permutation(E)[:K] for _ in range(T)]) if T else \
            np.zeros((0, K), np.int64)
        off, srt, pos = O.permute(ids, E)
        flat = ids.reshape(-1)
        assert sorted(srt.tolist()) == list(range(T * K))
        assert all(flat[srt[i]] <= flat[srt[i + 1]] for i in range(T * K - 1))
        cnt = [0] * E
        for e in flat:
            cnt[e] += 1
        assert off.tolist() == [sum(cnt[:e]) for e in range(E + 1)]
        assert all(pos[srt[i]] == i for i in range(T * K))
        for e in range(E):
            seg = srt[off[e]:off[e + 1]].tolist()
            assert seg == sorted(seg) and all(flat[x] == e for x in seg)


def pin_combine_bruteforce():
    r = _rng(11)
    T, K, H = 5, 3, 4
    y = r.standard_normal((T * K, H))
    w = r.standard_normal((T, K))
    pos = r.permutation(T * K)
    out = O.combine(y, w, pos, 1.5, "f64")
    for t in range(T):
        for h in range(H):
            want = 1.5 * math.fsum(w[t, k] * y[pos[t * K + k], h] for k in range(K))
            assert abs(out[t, h] - want) < 1e-13


def pin_ffn_soft_mixture():
    """K = E with softmax and no renormalization is the dense soft mixture
    sum_e p_e f_e(x); the routed path must reproduce it."""
    r = _rng(12)
    T, H, E, F = 6, 12, 4, 5
    x = _f32(r.standard_normal((T, H)))
    z = _f32(r.standard_normal((T, E)))
    wgu = _f32(r.standard_normal((E, 2 * F, H)) * 0.3)
    wd = _f32(r.standard_normal((E, H, F)) * 0.3)
    bgu = _f32(r.standard_normal((E, 2 * F)) * 0.1)
    bd = _f32(r.standard_normal((E, H)) * 0.1)
    for act in ("silu_and_mul", "swigluoai"):
        got = O.moe_ffn_forward(x, z, wgu, wd, top_k=E, renormalize=False, act=act,
                                dtype="f32", b_gate_up=bgu, b_down=bd)["out"]
        p = np.exp(z - z.max(1, keepdims=True))
        p = p / p.sum(1, keepdims=True)
        want = np.zeros((T, H))
        for t in range(T):
            for e in range(E):
                layout, al, be, li, _ = O.ACTIVATIONS[act]
                h = wgu[e] @ x[t] + bgu[e]
                g, u = (h[:F], h[F:]) if layout == "stacked" else (h[0::2], h[1::2])
                if li > 0:
                    g, u = np.minimum(g, li), np.clip(u, -li, li)
                a = _f32(g / (1 + np.exp(-al * g)) * (u + be))
                want[t] += _f32(p[t, e]) * (wd[e] @ a + bd[e])
        assert np.allclose(got, want, rtol=2e-6, atol=1e-6), act


def pin_ffn_token_subset():
    r = _rng(13)
    T, H, E, F, K = 20, 8, 6, 4, 2
    x = _f32(r.standard_normal((T, H)))
    z = _f32(r.standard_normal((T, E)))
    wgu = _f32(r.standard_normal((E, 2 * F, H)) * 0.3)
    wd = _f32(r.standard_normal((E, H, F)) * 0.3)
    kw = dict(top_k=K, scoring="sigmoid", renormalize=True, routed_scaling_factor=2.5,
              num_expert_group=3, topk_group=2, correction_bias=_f32(r.uniform(-.1, .1, E)),
              dtype="bf16")
    full = O.moe_ffn_forward(x, z, wgu, wd, **kw)["out"]
    sub = O.moe_ffn_forward(x, z, wgu, wd, tokens=np.array([17, 3, 9]), **kw)["out"]
    assert np.array_equal(sub, full[[17, 3, 9]])


def pin_dispatch_rule():
    d = GOLDEN["indexed_dispatch"]
    assert d["H_multiple"] == 128 and d["F_multiple"] == 256
    assert O.indexed_backend_applies(16, 8, 256, 7168, 2048, "silu_and_mul", False)
    assert not O.indexed_backend_applies(4096, 8, 128, 2048, 768, "silu_and_mul", False)
    assert not O.indexed_backend_applies(16, 4, 128, 2880, 2880, "swigluoai", True)
    assert O.indexed_backend_applies(64, 8, 256, 7168, 2048, "silu_and_mul", False)
    assert not O.indexed_backend_applies(65, 8, 256, 7168, 2048, "silu_and_mul", False)
    assert not O.indexed_backend_applies(16, 8, 256, 7168 + 64, 2048, "silu_and_mul", False)
    assert not O.indexed_backend_applies(16, 8, 256, 7168, 2048 + 128, "silu_and_mul", False)


# ------------------------------------------------------------------- FP8 grouped GEMM
def pin_e4m3fn_decode():
    """All 256 codes against torch's float8_e4m3fn, plus the format's landmarks."""
    codes = np.arange(256, dtype=np.uint8)
    got = O.decode_e4m3fn(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, want, equal_nan=True)
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0      # largest finite
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9  # min normal, min subnormal
    assert got[0x38] == 1.0 and got[0x00] == 0.0 and np.signbit(got[0x80])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isnan(got).sum() == 2


def _fp8_case(seed, E, max_m, K, N):
    r = _rng(seed)
    a = r.integers(0, 256, (E, max_m, K), dtype=np.uint8)
    b = r.integers(0, 256, (E, N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38  # no NaN codes in operands
    b[(b & 0x7F) == 0x7F] = 0x30
    sa = r.uniform(0.25, 4.0, (E, max_m, K // 128))
    sb = r.uniform(0.25, 4.0, (E, N // 128, K // 128))
    return a, sa, b, sb


def pin_fp8_gemm_dequantized_bruteforce():
    """The page's accuracy reference: dequantize both operands under their scales
    (every element times its own row / block scale), then one plain product per expert,
    in torch float64; the oracle's block-wise order must agree to one bf16 step."""
    E, max_m, K, N = 2, 5, 256, 256
    a, sa, b, sb = _fp8_case(21, E, max_m, K, N)
    counts = np.array([5, 3])
    out = O.grouped_gemm_fp8_masked(a, sa, b, sb, counts)
    A = torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64)
    B = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64)
    ka = torch.arange(K) // 128
    for g in range(E):
        deq_a = A[g] * torch.from_numpy(sa[g])[:, ka]
        nb = torch.arange(N) // 128
        deq_b = B[g] * torch.from_numpy(sb[g])[nb][:, ka]
        want = (deq_a @ deq_b.T).numpy()
        m = counts[g]
        got = out[g, :m]
        ulp = np.abs(O.round_to(want[:m], "bf16")) * 2.0 ** -7
        assert np.all(np.abs(got - want[:m]) <= ulp + 1e-300)
        assert np.isnan(out[g, m:]).all()


def pin_fp8_gemm_exact_integers():
    """Small integer codes and power-of-two scales: every product and partial sum is an
    exact integer multiple of the scale, so the result equals an integer matmul."""
    r = _rng(22)
    E, max_m, K, N = 2, 4, 256, 128
    vals = np.array([-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0])
    ia = r.integers(0, vals.size, (E, max_m, K))
    ib = r.integers(0, vals.size, (E, N, K))
    enc = torch.tensor(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a, b = enc[ia], enc[ib]
    sa = np.full((E, max_m, K // 128), 0.5)
    sb = np.full((E, N // 128, K // 128), 4.0)
    out = O.grouped_gemm_fp8_masked(a, sa, b, sb, np.array([max_m, max_m]))
    for g in range(E):
        want = (vals[ia[g]].astype(np.int64) @ vals[ib[g]].astype(np.int64).T) * 2.0
        assert np.array_equal(out[g], O.round_to(want.astype(np.float64), "bf16"))
    assert abs(O.round_to(np.array([257.0]), "bf16")[0] - 256.0) == 0  # the cast is real


def pin_fp8_count_clamp():
    """A count past max_m is read as max_m, a negative one as 0."""
    E, max_m, K, N = 4, 3, 128, 128
    a, sa, b, sb = _fp8_case(23, E, max_m, K, N)
    out = O.grouped_gemm_fp8_masked(a, sa, b, sb, np.array([-2, 0, max_m + 5, 2]))
    assert np.isnan(out[0]).all() and np.isnan(out[1]).all()
    assert not np.isnan(out[2]).any()
    assert not np.isnan(out[3, :2]).any() and np.isnan(out[3, 2:]).all()
    full = O.grouped_gemm_fp8_masked(a, sa, b, sb, np.array([max_m] * E))
    assert np.array_equal(out[2], full[2])


# ------------------------------------------------------- gelu_and_mul, SwiGLU op
PHI = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                  "normal_cdf_table.json")))["phi"]


def pin_gelu_table():
    """GELU(x) = x Phi(x) against the tabulated normal distribution function (15 decimals):
    separates the exact form from the tanh approximation (off by 1.5e-4 at x = 1)."""
    for xs, phi in PHI.items():
        x = float(xs)
        for v, want in ((x, x * phi), (-x, -x * (1.0 - phi))):
            got = float(O.gelu(np.array([v]))[0])
            assert abs(got - want) <= 2e-15 * max(1.0, abs(want)), (v, got, want)
    assert float(O.gelu(np.array([0.0]))[0]) == 0.0


def pin_gelu_torch_and_symmetry():
    """Against torch's exact GELU in float64, and GELU(x) - GELU(-x) = x."""
    x = _rng(21).standard_normal(4000) * 4
    got = O.gelu(x)
    want = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(got, want, rtol=1e-14, atol=1e-15)
    assert np.allclose(got - O.gelu(-x), x, rtol=0, atol=1e-12)


def pin_gelu_and_mul_gemm():
    """gelu_and_mul over a stacked gate_up: act(x Wg^T + bg) * (x Wu^T + bu) per expert,
    with torch's exact GELU as the activation (brute-force product per expert)."""
    r = _rng(22)
    E, F, K = 3, 5, 7
    off = np.array([0, 4, 4, 9])
    a = _f32(r.standard_normal((9, K)))
    b = _f32(r.standard_normal((E, 2 * F, K)))
    bias = _f32(r.standard_normal((E, 2 * F)) * 0.1)
    got = O.grouped_gemm_act(a, b, off, "gelu_and_mul", bias, "f64")
    want = np.zeros((9, F))
    for e in range(E):
        for m in range(off[e], off[e + 1]):
            h = torch.from_numpy(b[e] @ a[m] + bias[e])
            want[m] = (torch.nn.functional.gelu(h[:F], approximate="none") * h[F:]).numpy()
    assert np.allclose(got, want, rtol=1e-13, atol=1e-14)
    assert O.ACTIVATIONS["gelu_and_mul"][0] == "stacked"


def pin_swiglu_op_forms():
    """[MR] SwiGLU op: separate gate/up, gate-then-up halves of one [.., 2F] input, and the
    interleaved [SPEC] fusion 1 arrangement give the same values; the result is the
    activation's closed form stored in the requested dtype."""
    r = _rng(23)
    g = _f32(r.standard_normal((6, 10)) * 4)
    u = _f32(r.standard_normal((6, 10)) * 4)
    for al, be, li in ((1.0, 0.0, 0.0), (1.702, 1.0, 7.0), (0.5, -0.25, 2.0)):
        sep = O.swiglu_op(g, u, al, be, li, out_dtype="f64")
        want = np.array([[float(_dswiglu(gi, ui, al, be, li)) for gi, ui in zip(gr, ur)]
                         for gr, ur in zip(g, u)])
        assert np.allclose(sep, want, rtol=1e-13, atol=1e-14)
        st = O.swiglu_op(np.concatenate([g, u], axis=1), None, al, be, li, out_dtype="f64")
        il = np.empty((6, 20))
        il[:, 0::2], il[:, 1::2] = g, u
        it = O.swiglu_op(il, None, al, be, li, fusion="interleaved", out_dtype="f64")
        assert np.array_equal(st, sep) and np.array_equal(it, sep)
        bf = O.swiglu_op(g, u, al, be, li, out_dtype="bf16")
        assert np.array_equal(bf, torch.from_numpy(sep).to(torch.bfloat16).double().numpy())


# ------------------------------------------------------------ padded / masked layouts
def _routes_by_expert(ids, E):
    return [[r for r in range(ids.size) if ids[r] == e] for e in range(E)]


def pin_permute_align_definition():
    """[TO] MoEPermuteAlignFwdOp's definition, checked entry by entry on random and
    degenerate ids: each expert's range holds exactly its routes once, padded with numel
    to a multiple of block_size; num_post_pad is the sum of the padded lengths; blocks
    name their owner; everything past the used length is numel / outside [0, E)."""
    r = _rng(31)
    for T, K, E, bs in ((50, 3, 7, 16), (1, 1, 4, 64), (64, 8, 16, 1), (9, 2, 3, 5),
                        (0, 2, 3, 4)):
        ids = r.integers(0, E, size=(T, K)) if T else np.zeros((0, K), dtype=np.int64)
        if T == 64:
            ids[:] = 5          # one expert takes everything
        flat = ids.reshape(-1)
        numel = flat.size
        st, blk, used = O.permute_align(ids, E, bs)
        assert len(st) == numel + (E + 1) * (bs - 1)
        assert len(blk) == -(-len(st) // bs)
        want_used = sum(-(-len(rt) // bs) * bs for rt in _routes_by_expert(flat, E))
        assert used == want_used and used % bs == 0
        assert np.all(st[used:] == numel)
        assert np.all((blk[used // bs:] < 0) | (blk[used // bs:] >= E))
        start = 0
        for e, rt in enumerate(_routes_by_expert(flat, E)):
            n = -(-len(rt) // bs) * bs
            seg = st[start:start + n]
            assert sorted(seg[seg < numel].tolist()) == rt
            assert np.all(seg[len(rt):] == numel)
            assert np.all(blk[start // bs:(start + n) // bs] == e)
            start += n


def pin_pre_permute_layouts():
    """Each layout puts hidden[r / K] at inverse[r]; the tight contiguous layout equals
    permute() plus a gather; masked slabs keep the first max_m routes of an expert (in
    route order) and drop the rest; per_row ids and segment ends describe the same rows."""
    r = _rng(32)
    T, K, E, H = 40, 3, 6, 5
    x = r.standard_normal((T, H))
    ids = r.integers(0, E, size=(T, K))
    ids[:20, 0] = 2                       # expert 2 overflows a small slab
    flat = ids.reshape(-1)
    off, srt, pos = O.permute(ids, E)
    for bs in (1, 4, 16):
        outc, ends, invc = O.pre_permute(x, ids, E, "contiguous", bs)
        outp, rowid, invp = O.pre_permute(x, ids, E, "per_row", bs)
        assert np.array_equal(invc, invp) and np.array_equal(outc[invc], x[np.arange(T * K) // K])
        for e in range(E):
            lo = ends[e - 1] if e else 0
            own = np.nonzero(rowid == e)[0]
            assert np.all((own >= lo) & (own < ends[e])) and own.size == np.sum(flat == e)
            assert (ends[e] - lo) % bs == 0
        if bs == 1:
            assert np.array_equal(invc, pos) and np.array_equal(ends, off[1:])
    max_m = 9
    outm, cnt, invm = O.pre_permute(x, ids, E, "masked", max_m=max_m)
    for e in range(E):
        rt = np.nonzero(flat == e)[0]
        assert cnt[e] == min(rt.size, max_m)
        assert np.array_equal(invm[rt[:max_m]], e * max_m + np.arange(cnt[e]))
        assert np.all(invm[rt[max_m:]] == -1)
    live = invm >= 0
    assert np.array_equal(outm.reshape(-1, H)[invm[live]], x[np.nonzero(live)[0] // K])


def pin_grouped_gemm_layouts():
    """One routed problem laid out three ways: every route's product row agrees across
    layouts and with a per-row brute-force dot product; uncovered rows are unspecified
    (NaN); masked counts past max_m or negative are clamped."""
    r = _rng(33)
    T, K, E, H, N = 30, 2, 5, 7, 6
    x = _f32(r.standard_normal((T, H)))
    ids = r.integers(0, E, size=(T, K))
    w = _f32(r.standard_normal((E, N, H)))
    bias = _f32(r.standard_normal((E, N)))
    flat = ids.reshape(-1)
    want = np.array([w[flat[q]] @ x[q // K] + bias[flat[q]] for q in range(T * K)])
    for lay, kw in (("contiguous", {"block_size": 4}), ("per_row", {"block_size": 8}),
                    ("masked", {"max_m": 64})):
        a, meta, inv = O.pre_permute(x, ids, E, lay, **kw)
        out = O.grouped_gemm_layout(np.nan_to_num(a), w, lay, meta, bias, None, "f64")
        flat_out = out.reshape(-1, N)
        assert np.allclose(flat_out[inv], want, rtol=1e-12, atol=1e-12), lay
        covered = np.zeros(flat_out.shape[0], bool)
        covered[inv] = True
        if lay != "contiguous":   # a contiguous segment also owns its pad rows
            assert np.all(np.isnan(flat_out[~covered]))
    # masked count clamping
    a = _f32(r.standard_normal((3, 4, H)))
    out = O.grouped_gemm_layout(a, w[:3], "masked", [9, -2, 2], None, None, "f64")
    assert np.all(np.isfinite(out[0])) and np.all(np.isnan(out[1]))
    assert np.all(np.isfinite(out[2, :2])) and np.all(np.isnan(out[2, 2:]))
    # activation on a layout: gated product of the same rows
    a, meta, inv = O.pre_permute(x, ids, E, "masked", max_m=64)
    w2 = _f32(r.standard_normal((E, 2 * N, H)))
    got = O.grouped_gemm_layout(a, w2, "masked", meta, None, "silu_and_mul", "f64")
    for q in range(T * K):
        h = w2[flat[q]] @ x[q // K]
        g, u = h[:N], h[N:]
        assert np.allclose(got.reshape(-1, N)[inv[q]], g / (1 + np.exp(-g)) * u, rtol=1e-12)


def pin_combine_negative_positions():
    """A route without a row (inverse -1) contributes nothing; the rest is the plain
    weighted sum (brute force)."""
    r = _rng(34)
    T, K, H = 6, 3, 4
    y = r.standard_normal((10, H))
    w = r.standard_normal((T, K))
    pos = r.integers(0, 10, size=(T, K))
    pos[1, 2] = -1
    pos[4, :] = -1
    got = O.combine(y, w, pos.reshape(-1), 1.5, "f64")
    for t in range(T):
        want = sum(w[t, k] * y[pos[t, k]] for k in range(K) if pos[t, k] >= 0)
        assert np.allclose(got[t], 1.5 * np.asarray(want, dtype=np.float64) if np.ndim(want) else np.zeros(H), atol=1e-14)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
