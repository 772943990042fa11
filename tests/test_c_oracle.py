"""The C oracle (oracle/moe_ref.c): the same pins as the numpy oracle, planted mistakes
in its source, and agreement with the numpy oracle on random cases.

The two oracles are written separately from the same pages; they share no code. Where
both are right they agree to the last bit except where float64 sums are taken in another
order (BLAS blocking against index order), which moves a stored value by at most one step
of its storage format.
"""
import inspect
import re

import numpy as np
import pytest

import oracle.moe_oracle as O
import oracle_pins as P
from oracle import build_ref
from oracle.c_oracle import COracle, load


@pytest.fixture(scope="module")
def C():
    return load(threads=4)


def _uses(pin):
    return set(re.findall(r"\bO\.(\w+)", inspect.getsource(pin)))


C_PINS = [p for p in P.ALL_PINS if all(hasattr(COracle, n) for n in _uses(p))]
NUMPY_ONLY = sorted(p.__name__ for p in P.ALL_PINS if p not in C_PINS)


def test_numpy_only_pins_are_the_layout_ops():
    # the C oracle leaves the padded / masked layout ops and the dispatch rule to numpy
    assert NUMPY_ONLY == ["pin_dispatch_rule", "pin_grouped_gemm_layouts",
                          "pin_permute_align_definition", "pin_pre_permute_layouts"]


@pytest.mark.parametrize("pin", C_PINS, ids=lambda f: f.__name__)
def test_c_pin(pin, C, monkeypatch):
    monkeypatch.setattr(P, "O", C)
    pin()


# (find, replace) in moe_ref.c; every mutant stays within its buffers.
C_MUTANTS = {
    "ties go to the higher index": ("(va == vb && a < b)", "(va == vb && a > b)"),
    "gate clamped from below too": ("    if (g > a->limit) g = a->limit;\n",
                                    "    if (g > a->limit) g = a->limit;\n"
                                    "    if (g < -a->limit) g = -a->limit;\n"),
    "limit 0 does not disable the clamp": ("if (a->limit > 0.0) {", "if (a->limit >= 0.0) {"),
    "scaling factor applied twice": (
        "moe_ref_round(wn * c->routed_scaling_factor, MOE_REF_F32)",
        "moe_ref_round(wn * c->routed_scaling_factor * c->routed_scaling_factor, MOE_REF_F32)"),
    "renormalized over all experts": ("for (int64_t k = 0; k < K; ++k) sum += s[ids[k]];",
                                      "for (int64_t k = 0; k < E; ++k) sum += s[k];"),
    "biased group score is the max": ("gs[g] = moe_ref_round(ug[b1] + ug[b2], MOE_REF_F32);",
                                      "gs[g] = ug[b1];"),
    "bias left out of the keys": (
        "u[e] = x->bias ? moe_ref_round(s32 + x->bias[e], MOE_REF_F32) : s32;", "u[e] = s32;"),
    "gate and up halves swapped": ("else { *gi = j; *ui = F + j; }",
                                   "else { *gi = F + j; *ui = j; }"),
    "interleaved pairs swapped": ("{ *gi = 2 * j; *ui = 2 * j + 1; }",
                                  "{ *gi = 2 * j + 1; *ui = 2 * j; }"),
    "activation not stored in the operand dtype": (
        "a[j] = moe_ref_round(moe_ref_gated(act, h[gi], h[ui]), act_fmt);",
        "a[j] = moe_ref_gated(act, h[gi], h[ui]);"),
    "rounding ties away from zero": ("ldexp(nearbyint(ldexp(x, -q)), q)",
                                     "ldexp(round(ldexp(x, -q)), q)"),
    "sigmoid sign flipped": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "sqrt_softplus without the root": ("s[e] = sqrt(fmax(z, 0.0) + log1p(exp(-fabs(z))));",
                                       "s[e] = fmax(z, 0.0) + log1p(exp(-fabs(z)));"),
    "float16 router fill is -1e30": ("fmt == MOE_REF_F16 ? -1.0e4 : -1.0e30",
                                     "fmt == MOE_REF_F16 ? -1.0e30 : -1.0e30"),
    "weight_scale without the scaling factor": (
        "moe_ref_round(routed_scaling_factor * local, fmt)", "moe_ref_round(local, fmt)"),
    "combine weights read transposed": ("topk_weights[t * K + k] *",
                                        "topk_weights[(k * T + t) % (T * K)] *"),
    "e4m3 subnormals off by a factor two": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e4m3 exponent bias 8": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    "fp8 b scale of the first K block": ("c->sb[(g * (N / 128) + n / 128) * nkb + kb]",
                                         "c->sb[(g * (N / 128) + n / 128) * nkb]"),
    "fp8 negative count read as its magnitude": ("if (cnt < 0) cnt = 0;",
                                                 "if (cnt < 0) cnt = -cnt;"),
    "down bias dropped": ("y[o] = bd ? acc + widen1(bd, fmt, e * N + o) : acc;", "y[o] = acc;"),
    "layer sums unweighted": ("acc[o] += w * y[o];", "acc[o] += y[o];"),
    "shared expert gate without its sigmoid": ("h[j] * sigmoid(h[j]) * h[S + j]",
                                               "h[j] * h[S + j]"),
    "gelu by its tanh approximation": (
        "0.5 * g * (1.0 + erf(g / sqrt(2.0))) * l",
        "0.5 * g * (1.0 + tanh(sqrt(2.0 / 3.141592653589793) * (g + 0.044715 * g * g * g))) * l"),
    "permute not stable": ("for (int64_t r = 0; r < R; ++r) {\n    const int64_t p = fill",
                           "for (int64_t r = R - 1; r >= 0; --r) {\n    const int64_t p = fill"),
}


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(name, tmp_path, monkeypatch):
    find, repl = C_MUTANTS[name]
    src = open(build_ref.SRC).read()
    assert src.count(find) == 1, f"mutation site not unique: {find!r}"
    path = tmp_path / "moe_ref.c"
    path.write_text(src.replace(find, repl))
    # a mutant may leave a parameter unused: warnings stay warnings here
    lib = build_ref.build(str(path), str(tmp_path / "libmutant.so"), extra=("-Wno-error",))
    monkeypatch.setattr(P, "O", COracle(lib, threads=2))
    for pin in C_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, TypeError):
            return
    pytest.fail(f"no pin catches the planted mistake: {name}")


# ----------------------------------------------------------------- agreement with numpy
def _ulp(v, fmt):
    bits = {"f32": 24, "bf16": 8, "f16": 11}[fmt]
    a = np.abs(np.asarray(v, np.float64))
    return np.ldexp(1.0, (np.frexp(np.maximum(a, 1e-30))[1] - bits))


def _close(a, b, fmt):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape
    ok = (a == b) | (np.abs(a - b) <= _ulp(np.maximum(np.abs(a), np.abs(b)), fmt))
    assert ok.all(), (np.argwhere(~ok)[:5], a[~ok][:5], b[~ok][:5])


ROUTES = [
    dict(E=16, K=4, scoring="softmax", renormalize=True, rsf=1.0),
    dict(E=32, K=8, scoring="sigmoid", renormalize=True, rsf=2.5, G=8, TG=4, bias=True),
    dict(E=24, K=3, scoring="sqrt_softplus", renormalize=False, rsf=1.5, G=4, TG=2),
    dict(E=8, K=2, scoring="sigmoid", renormalize=True, rsf=1.0, G=8, TG=3, bias=True),
]


@pytest.mark.parametrize("case", range(len(ROUTES)))
def test_route_matches_numpy(case, C):
    c = ROUTES[case]
    r = np.random.default_rng(100 + case)
    T = 300
    z = r.standard_normal((T, c["E"])).astype(np.float32)
    bias = r.uniform(-0.1, 0.1, c["E"]).astype(np.float32) if c.get("bias") else None
    kw = dict(top_k=c["K"], scoring=c["scoring"], renormalize=c["renormalize"],
              routed_scaling_factor=c["rsf"], num_expert_group=c.get("G", 1),
              topk_group=c.get("TG", 1), correction_bias=bias, local_expert_start=4,
              local_expert_count=c["E"] // 2, router_probs_dtype="bf16")
    a, b = O.route(z, **kw), C.route(z, **kw)
    # selection compares the same float32 keys, so ids agree wherever the keys do
    assert np.array_equal(a.keys, b.keys)
    if a.group_scores is not None:
        assert np.array_equal(a.group_scores, b.group_scores)
    assert np.array_equal(a.topk_ids, b.topk_ids)
    assert np.array_equal(a.gap_sel, b.gap_sel) and np.array_equal(a.gap_group, b.gap_group)
    assert np.allclose(a.scores, b.scores, rtol=1e-15, atol=0)
    assert np.allclose(a.wn, b.wn, rtol=1e-15, atol=0)
    _close(a.topk_weights, b.topk_weights, "f32")
    _close(a.router_probs, b.router_probs, "bf16")
    _close(a.weight_scale, b.weight_scale, "bf16")


LAYERS = [
    dict(T=40, H=64, E=8, F=32, K=2, act="silu_and_mul", dtype="bf16"),
    dict(T=24, H=48, E=6, F=24, K=2, act="swigluoai", dtype="bf16", bias=True),
    dict(T=20, H=32, E=16, F=16, K=4, act="gelu_and_mul", dtype="f16", scoring="sigmoid",
         G=4, TG=2, cbias=True, rsf=2.5, S=24),
    dict(T=16, H=40, E=4, F=20, K=1, act="silu_and_mul", dtype="f32", scoring="sqrt_softplus"),
]


@pytest.mark.parametrize("case", range(len(LAYERS)))
def test_layer_matches_numpy(case, C):
    import torch
    c = LAYERS[case]
    r = np.random.default_rng(200 + case)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[c["dtype"]]

    def t(shape, scale):
        return torch.from_numpy(r.standard_normal(shape) * scale).to(tdt)
    T, H, E, F, K = c["T"], c["H"], c["E"], c["F"], c["K"]
    x, z = t((T, H), 1.0), torch.from_numpy(r.standard_normal((T, E)).astype(np.float32))
    wgu, wd = t((E, 2 * F, H), 0.2), t((E, H, F), 0.2)
    bgu, bd = (t((E, 2 * F), 0.05), t((E, H), 0.05)) if c.get("bias") else (None, None)
    S = c.get("S", 0)
    swgu, swd = (t((2 * S, H), 0.2), t((H, S), 0.2)) if S else (None, None)
    cb = r.uniform(-0.1, 0.1, E).astype(np.float32) if c.get("cbias") else None
    kw = dict(top_k=K, scoring=c.get("scoring", "softmax"), renormalize=True,
              routed_scaling_factor=c.get("rsf", 1.0), num_expert_group=c.get("G", 1),
              topk_group=c.get("TG", 1), act=c["act"], dtype=c["dtype"], correction_bias=cb,
              b_gate_up=bgu, b_down=bd, shared_w_gate_up=swgu, shared_w_down=swd)

    def f64(v):
        return None if v is None else v.to(torch.float64).numpy()
    a = O.moe_ffn_forward(f64(x), z.numpy(), f64(wgu), f64(wd), **{
        **kw, "b_gate_up": f64(bgu), "b_down": f64(bd), "shared_w_gate_up": f64(swgu),
        "shared_w_down": f64(swd)})
    b = C.moe_ffn_forward(x, z, wgu, wd, **kw)      # storage-format inputs, widened in C
    assert np.array_equal(a["route"].topk_ids, b["route"].topk_ids)
    _close(a["out"], b["out"], c["dtype"])
    if S:
        _close(a["shared_out"], b["shared_out"], c["dtype"])
    sub = C.moe_ffn_forward(x, z, wgu, wd, tokens=np.array([T - 1, 0, 5]), **kw)
    assert np.array_equal(sub["out"], b["out"][[T - 1, 0, 5]])


def test_fp8_matches_numpy(C):
    a, sa, b, sb = P._fp8_case(41, 3, 9, 384, 256)
    counts = np.array([9, 0, -2])
    x, y = O.grouped_gemm_fp8_masked(a, sa, b, sb, counts), \
        C.grouped_gemm_fp8_masked(a, sa, b, sb, counts)
    assert np.array_equal(np.isnan(x), np.isnan(y))
    m = ~np.isnan(x)
    _close(x[m], y[m], "bf16")


def test_threads_do_not_change_results(C):
    r = np.random.default_rng(7)
    x = r.standard_normal((33, 16))
    z = r.standard_normal((33, 8))
    wgu = r.standard_normal((8, 24, 16)) * 0.3
    wd = r.standard_normal((8, 16, 12)) * 0.3
    kw = dict(top_k=2, renormalize=True, dtype="bf16")
    one = COracle(C.path, threads=1).moe_ffn_forward(x, z, wgu, wd, **kw)["out"]
    many = COracle(C.path, threads=5).moe_ffn_forward(x, z, wgu, wd, **kw)["out"]
    assert np.array_equal(one, many)


def test_bad_arguments_raise(C):
    with pytest.raises(ValueError):
        C.route(np.zeros((2, 6)), 3, num_expert_group=4, topk_group=1)   # E % G != 0
    with pytest.raises(ValueError):
        C.route(np.zeros((2, 8)), 2, expert_ids=np.array([[0, 8], [1, 2]]))
    with pytest.raises(ValueError):
        C.permute(np.array([[0, 5]]), 4)
