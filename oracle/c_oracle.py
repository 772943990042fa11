"""ctypes front end of the C float64 oracle (moe_ref.c), with the numpy oracle's names.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg are the only callers. It loads oracle/_build/libmoe_ref.so (built by
oracle/build_ref.py from moe_ref.c alone) and never the GPU library.

COracle exposes the subset of moe_oracle's functions that the C code implements, with
the same signatures and results, so the same pins run against both oracles. Every
arithmetic step runs in C; this file only converts arrays (storage-format codes,
contiguous copies) and splits a fused [.., 2F] array for swiglu_op.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libmoe_ref.so")

F64, F32, BF16, F16 = 0, 1, 2, 3
FMT_CODE = {"f64": F64, "f32": F32, "bf16": BF16, "f16": F16}
SCORING = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2}
LAYOUT = {"stacked": 0, "interleaved": 1}
KIND = {"swiglu": 0, "gelu": 1}

# name -> (row layout of gate_up, alpha, beta, limit, kind).  [TO] MoEGroupedGemmFwdOp:
# silu_and_mul and gelu_and_mul read gate rows then up rows; swigluoai reads interleaved
# rows with the constants 1.702, 1, 7.
ACTIVATIONS = {
    "silu_and_mul": ("stacked", 1.0, 0.0, 0.0, "swiglu"),
    "swigluoai": ("interleaved", 1.702, 1.0, 7.0, "swiglu"),
    "gelu_and_mul": ("stacked", 0.0, 0.0, 0.0, "gelu"),
}


class _Act(C.Structure):
    _fields_ = [("layout", C.c_int32), ("kind", C.c_int32), ("alpha", C.c_double),
                ("beta", C.c_double), ("limit", C.c_double)]


class _RouteCfg(C.Structure):
    _fields_ = [("E", C.c_int64), ("K", C.c_int64), ("scoring", C.c_int32),
                ("renormalize", C.c_int32), ("routed_scaling_factor", C.c_double),
                ("num_expert_group", C.c_int64), ("topk_group", C.c_int64)]


class _FfnCfg(C.Structure):
    _fields_ = [("H", C.c_int64), ("F", C.c_int64), ("S", C.c_int64), ("route", _RouteCfg),
                ("act", _Act), ("fmt", C.c_int32), ("dtype", C.c_int32)]


@dataclass
class RouteResult:
    scores: np.ndarray
    topk_ids: np.ndarray
    wn: np.ndarray
    topk_weights: np.ndarray
    gap_sel: np.ndarray
    gap_group: np.ndarray
    router_probs: Optional[np.ndarray] = None
    weight_scale: Optional[np.ndarray] = None
    keys: Optional[np.ndarray] = None
    group_scores: Optional[np.ndarray] = None


def _stored(x):
    """(contiguous host array, format code) of a numpy array or a CPU torch tensor; 16-bit
    floats are passed as their bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            t = x.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            if t.dtype == torch.float16:
                return t.view(torch.int16).numpy().view(np.uint16), F16
            if t.dtype == torch.float32:
                return t.numpy(), F32
            return t.to(torch.float64).numpy(), F64
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype == np.float16:
        return np.ascontiguousarray(a).view(np.uint16), F16
    if a.dtype == np.float32:
        return np.ascontiguousarray(a), F32
    return np.ascontiguousarray(a, dtype=np.float64), F64


def _same_fmt(arrays):
    """Bring optional arrays to one storage format (float64 when they differ)."""
    got = [None if a is None else _stored(a) for a in arrays]
    fmts = {g[1] for g in got if g is not None}
    if len(fmts) <= 1:
        fmt = fmts.pop() if fmts else F64
        return [None if g is None else g[0] for g in got], fmt
    return [None if a is None else np.ascontiguousarray(np.asarray(_as_f64(a)))
            for a in arrays], F64


def _as_f64(x):
    a, fmt = _stored(x)
    if fmt == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if fmt == F16:
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _act(act):
    if isinstance(act, str):
        act = ACTIVATIONS[act]
    act = tuple(act)
    if len(act) == 4:
        act = act + ("swiglu",)
    layout, alpha, beta, limit, kind = act
    return _Act(LAYOUT[layout], KIND[kind], float(alpha), float(beta), float(limit))


class COracle:
    """The C oracle behind the numpy oracle's function names (see module docstring)."""

    ACTIVATIONS = ACTIVATIONS

    def __init__(self, path: str = LIB_PATH, threads: int = 1):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run oracle/build_ref.py (or "
                               "__graft_entry__.build()) first")
        self.path = path
        self.lib = L = C.CDLL(path)
        vp, i64, i32, dbl = C.c_void_p, C.c_int64, C.c_int32, C.c_double
        L.moe_ref_last_error.restype = C.c_char_p
        L.moe_ref_set_threads.argtypes = [C.c_int]
        L.moe_ref_round.restype = dbl
        L.moe_ref_round.argtypes = [dbl, i32]
        L.moe_ref_round_array.argtypes = [vp, i64, i32, vp]
        L.moe_ref_scores.argtypes = [vp, i32, i64, i64, i32, vp]
        L.moe_ref_ranked.argtypes = [vp, i64, vp]
        L.moe_ref_route.argtypes = [C.POINTER(_RouteCfg), vp, i32, i64, vp, vp] + [vp] * 8
        L.moe_ref_select_experts.argtypes = [C.POINTER(_RouteCfg), vp, i64, vp, vp, vp, vp]
        L.moe_ref_ep_outputs.argtypes = [vp, vp, i64, i64, dbl, i64, i64, i32, vp, vp]
        L.moe_ref_gated_array.argtypes = [C.POINTER(_Act), vp, vp, i64, vp]
        L.moe_ref_expert_mlp.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, i32,
                                         C.POINTER(_Act), i32, vp, vp]
        L.moe_ref_grouped_gemm.argtypes = [vp, i64, i64, vp, vp, i64, i64, vp, i32,
                                           C.POINTER(_Act), i32, vp]
        L.moe_ref_permute.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        L.moe_ref_combine.argtypes = [vp, i32, i64, vp, vp, i64, i64, i64, dbl, i32, vp]
        L.moe_ref_shared_expert.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, vp]
        L.moe_ref_ffn_forward.argtypes = [C.POINTER(_FfnCfg), vp, i64, vp, i32, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp, i64, vp, vp, vp, vp]
        L.moe_ref_decode_e4m3fn.argtypes = [vp, i64, vp]
        L.moe_ref_grouped_gemm_fp8_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                      vp]
        self.set_threads(threads)

    def set_threads(self, n: int) -> int:
        return self.lib.moe_ref_set_threads(int(n))

    def _check(self, rc):
        if rc != 0:
            raise ValueError(self.lib.moe_ref_last_error().decode())

    # ----------------------------------------------------------------- rounding
    def round_to(self, x, fmt: str) -> np.ndarray:
        a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty_like(a)
        self.lib.moe_ref_round_array(_p(a), a.size, FMT_CODE[fmt], _p(out))
        return out

    # ----------------------------------------------------------------- router
    def scores(self, logits, scoring: str) -> np.ndarray:
        z, fmt = _stored(logits)
        T, E = z.shape
        out = np.empty((T, E))
        self._check(self.lib.moe_ref_scores(_p(z), fmt, T, E, SCORING[scoring], _p(out)))
        return out

    def ranked(self, values) -> np.ndarray:
        v = np.ascontiguousarray(np.asarray(values, dtype=np.float64).reshape(-1))
        out = np.empty(v.size, dtype=np.int64)
        self.lib.moe_ref_ranked(_p(v), v.size, _p(out))
        return out

    @staticmethod
    def _rcfg(E, top_k, scoring="softmax", renormalize=False, rsf=1.0, G=1, TG=1):
        return _RouteCfg(E, int(top_k), SCORING[scoring], int(bool(renormalize)), float(rsf),
                         int(G), int(TG))

    def select_experts(self, s, top_k: int, correction_bias=None, num_expert_group: int = 1,
                       topk_group: int = 1):
        s = np.ascontiguousarray(np.asarray(s, dtype=np.float64))
        T, E = s.shape
        cfg = self._rcfg(E, top_k, G=num_expert_group, TG=topk_group)
        bias = None if correction_bias is None else \
            np.ascontiguousarray(np.asarray(correction_bias, dtype=np.float64))
        ids = np.empty((T, top_k), dtype=np.int64)
        gs, gg = np.empty(T), np.empty(T)
        self._check(self.lib.moe_ref_select_experts(C.byref(cfg), _p(s), T, _p(bias), _p(ids),
                                                     _p(gs), _p(gg)))
        return ids, gs, gg

    def route(self, logits, top_k: int, scoring: str = "softmax", renormalize: bool = False,
              routed_scaling_factor: float = 1.0, num_expert_group: int = 1,
              topk_group: int = 1, correction_bias=None, expert_ids=None,
              local_expert_start: int = 0, local_expert_count: Optional[int] = None,
              router_probs_dtype: Optional[str] = None) -> RouteResult:
        z, fmt = _stored(logits)
        return self._route(z, fmt, top_k, scoring, renormalize, routed_scaling_factor,
                           num_expert_group, topk_group, correction_bias, expert_ids,
                           local_expert_start, local_expert_count, router_probs_dtype)

    def _route(self, z, fmt, top_k, scoring="softmax", renormalize=False,
               routed_scaling_factor=1.0, num_expert_group=1, topk_group=1,
               correction_bias=None, expert_ids=None, local_expert_start=0,
               local_expert_count=None, router_probs_dtype=None):
        z = np.ascontiguousarray(z)
        T, E = z.shape
        K, G = int(top_k), int(num_expert_group)
        cfg = self._rcfg(E, K, scoring, renormalize, routed_scaling_factor, G, topk_group)
        bias = None if correction_bias is None else \
            np.ascontiguousarray(np.asarray(correction_bias, dtype=np.float64))
        ids_in = None if expert_ids is None else \
            np.ascontiguousarray(np.asarray(expert_ids, dtype=np.int64).reshape(T, K))
        sc, keys = np.empty((T, E)), np.empty((T, E))
        ids = np.empty((T, K), dtype=np.int64)
        wn, w = np.empty((T, K)), np.empty((T, K))
        gsc = np.empty((T, G)) if G > 1 else None
        gap_s, gap_g = np.empty(T), np.empty(T)
        self._check(self.lib.moe_ref_route(C.byref(cfg), _p(z), fmt, T, _p(bias), _p(ids_in),
                                           _p(sc), _p(ids), _p(wn), _p(w), _p(keys), _p(gsc),
                                           _p(gap_s), _p(gap_g)))
        res = RouteResult(sc, ids, wn, w, gap_s, gap_g, keys=keys, group_scores=gsc)
        if router_probs_dtype is not None:
            count = E - local_expert_start if local_expert_count is None else local_expert_count
            rp, ws = np.empty((T, count)), np.empty(T)
            self._check(self.lib.moe_ref_ep_outputs(
                _p(ids), _p(wn), T, K, float(routed_scaling_factor), int(local_expert_start),
                int(count), FMT_CODE[router_probs_dtype], _p(rp), _p(ws)))
            res.router_probs, res.weight_scale = rp, ws
        return res

    # ----------------------------------------------------------------- activation
    def _gated(self, act, g, l):
        g = np.asarray(g, dtype=np.float64)
        l = np.asarray(l, dtype=np.float64)
        shape = np.broadcast_shapes(g.shape, l.shape)
        g = np.ascontiguousarray(np.broadcast_to(g, shape)).reshape(-1)
        l = np.ascontiguousarray(np.broadcast_to(l, shape)).reshape(-1)
        out = np.empty(g.size)
        a = _act(act)
        self.lib.moe_ref_gated_array(C.byref(a), _p(g), _p(l), g.size, _p(out))
        return out.reshape(shape)

    def swiglu(self, g, l, alpha: float = 1.0, beta: float = 0.0, limit: float = 0.0):
        return self._gated(("stacked", alpha, beta, limit, "swiglu"), g, l)

    def gelu(self, x):
        return self._gated(("stacked", 0.0, 0.0, 0.0, "gelu"), x, 1.0)

    def gated(self, g, l, params):
        return self._gated(params, g, l)

    def swiglu_op(self, gate, up=None, alpha: float = 1.0, beta: float = 0.0,
                  limit: float = 0.0, fusion: str = "stacked", out_dtype: str = "f32"):
        gate = np.asarray(gate, dtype=np.float64)
        if up is None:
            F = gate.shape[-1] // 2
            if fusion == "stacked":
                gate, up = gate[..., :F], gate[..., F:]
            elif fusion == "interleaved":
                gate, up = gate[..., 0::2], gate[..., 1::2]
            else:
                raise ValueError(f"unknown layout {fusion!r}")
        return self.round_to(self.swiglu(gate, up, alpha, beta, limit), out_dtype)

    # ----------------------------------------------------------------- experts and stages
    def expert_mlp(self, x, w_gate_up, w_down, b_gate_up=None, b_down=None,
                   act="silu_and_mul", act_dtype: str = "f32"):
        (x, wgu, wd, bgu, bd), fmt = _same_fmt([x, w_gate_up, w_down, b_gate_up, b_down])
        M, H = x.shape
        N, F = wd.shape
        a, y = np.empty((M, F)), np.empty((M, N))
        ac = _act(act)
        self._check(self.lib.moe_ref_expert_mlp(_p(x), M, H, F, N, _p(wgu), _p(wd), _p(bgu),
                                                _p(bd), fmt, C.byref(ac), FMT_CODE[act_dtype],
                                                _p(a), _p(y)))
        return a, y

    def _grouped(self, a, b, expert_offsets, bias, act, out_dtype):
        (a, b, bias), fmt = _same_fmt([a, b, bias])
        M, K = a.shape
        E, N = b.shape[0], b.shape[1]
        off = np.ascontiguousarray(np.asarray(expert_offsets, dtype=np.int64))
        out = np.empty((M, N // 2 if act is not None else N))
        ac = None if act is None else _act(act)
        self._check(self.lib.moe_ref_grouped_gemm(
            _p(a), M, K, _p(b), _p(bias), E, N, _p(off), fmt,
            None if ac is None else C.byref(ac), FMT_CODE[out_dtype], _p(out)))
        return out

    def grouped_gemm(self, a, b, expert_offsets, bias=None, out_dtype: str = "f32"):
        return self._grouped(a, b, expert_offsets, bias, None, out_dtype)

    def grouped_gemm_act(self, a, b, expert_offsets, act="silu_and_mul", bias=None,
                         out_dtype: str = "f32"):
        return self._grouped(a, b, expert_offsets, bias, act, out_dtype)

    def permute(self, topk_ids, num_experts: int):
        ids = np.ascontiguousarray(np.asarray(topk_ids, dtype=np.int64))
        ids2 = ids.reshape(-1, ids.shape[-1]) if ids.ndim > 1 else ids.reshape(-1, 1)
        T, K = ids2.shape
        off = np.empty(num_experts + 1, dtype=np.int64)
        srt, pos = np.empty(T * K, dtype=np.int64), np.empty(T * K, dtype=np.int64)
        self._check(self.lib.moe_ref_permute(_p(ids2), T, K, num_experts, _p(off), _p(srt),
                                             _p(pos)))
        return off, srt, pos

    def combine(self, y, topk_weights, route_pos, scale: float = 1.0, out_dtype: str = "f32"):
        w = np.ascontiguousarray(np.asarray(topk_weights, dtype=np.float64))
        T, K = w.shape
        ya, fmt = _stored(y)
        ya = ya.reshape(-1, ya.shape[-1])
        pos = np.ascontiguousarray(np.asarray(route_pos, dtype=np.int64).reshape(-1))
        H = ya.shape[1]
        out = np.empty((T, H))
        self._check(self.lib.moe_ref_combine(_p(ya), fmt, ya.shape[0], _p(w), _p(pos), T, K,
                                             H, float(scale), FMT_CODE[out_dtype], _p(out)))
        return out

    def shared_expert_mlp(self, x, w_gate_up, w_down, dtype: str) -> np.ndarray:
        (x, wgu, wd), fmt = _same_fmt([x, w_gate_up, w_down])
        M, H = x.shape
        S = wgu.shape[0] // 2
        out = np.empty((M, H))
        self._check(self.lib.moe_ref_shared_expert(_p(x), M, H, S, _p(wgu), _p(wd), fmt,
                                                   FMT_CODE[dtype], _p(out)))
        return out

    def moe_ffn_forward(self, hidden, logits, w_gate_up, w_down, *, top_k: int,
                        scoring: str = "softmax", renormalize: bool = False,
                        routed_scaling_factor: float = 1.0, num_expert_group: int = 1,
                        topk_group: int = 1, act="silu_and_mul", dtype: str = "bf16",
                        correction_bias=None, expert_ids=None, b_gate_up=None, b_down=None,
                        shared_w_gate_up=None, shared_w_down=None, tokens=None):
        (x, wgu, wd, bgu, bd, swgu, swd), fmt = _same_fmt(
            [hidden, w_gate_up, w_down, b_gate_up, b_down, shared_w_gate_up, shared_w_down])
        z, zfmt = _stored(logits)
        T, H = x.shape
        E, F = wgu.shape[0], wd.shape[2]
        K = int(top_k)
        S = 0 if swgu is None else swgu.shape[0] // 2
        cfg = _FfnCfg(H, F, S, self._rcfg(E, K, scoring, renormalize, routed_scaling_factor,
                                          num_expert_group, topk_group), _act(act), fmt,
                      FMT_CODE[dtype])
        tok = np.arange(T, dtype=np.int64) if tokens is None else \
            np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        n = tok.size
        bias = None if correction_bias is None else \
            np.ascontiguousarray(np.asarray(correction_bias, dtype=np.float64))
        ids_in = None if expert_ids is None else \
            np.ascontiguousarray(np.asarray(expert_ids, dtype=np.int64).reshape(T, K))
        ids, w = np.empty((n, K), dtype=np.int64), np.empty((n, K))
        out = np.empty((n, H))
        sh = np.empty((n, H)) if S else None
        self._check(self.lib.moe_ref_ffn_forward(
            C.byref(cfg), _p(x), T, _p(z), zfmt, _p(bias), _p(ids_in), _p(wgu), _p(wd),
            _p(bgu), _p(bd), _p(swgu), _p(swd), _p(tok), n, _p(ids), _p(w), _p(out), _p(sh)))
        r = self._route(z[tok], zfmt, K, scoring, renormalize, routed_scaling_factor,
                       num_expert_group, topk_group, correction_bias,
                       None if ids_in is None else ids_in[tok])
        if not (np.array_equal(r.topk_ids, ids) and np.array_equal(r.topk_weights, w)):
            raise AssertionError("layer and router disagree on the routing")
        result = {"out": out, "route": r, "tokens": tok}
        if S:
            result["shared_out"] = sh
        return result

    # ----------------------------------------------------------------- FP8
    def decode_e4m3fn(self, codes) -> np.ndarray:
        c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
        out = np.empty(c.shape)
        self.lib.moe_ref_decode_e4m3fn(_p(c), c.size, _p(out))
        return out

    def grouped_gemm_fp8_masked(self, a_codes, a_scale, b_codes, b_scale, counts):
        a = np.ascontiguousarray(np.asarray(a_codes, dtype=np.uint8))
        b = np.ascontiguousarray(np.asarray(b_codes, dtype=np.uint8))
        sa = np.ascontiguousarray(np.asarray(a_scale, dtype=np.float64))
        sb = np.ascontiguousarray(np.asarray(b_scale, dtype=np.float64))
        cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int64))
        E, max_m, K = a.shape
        N = b.shape[1]
        out = np.empty((E, max_m, N))
        self._check(self.lib.moe_ref_grouped_gemm_fp8_masked(
            _p(a), _p(sa), _p(b), _p(sb), _p(cnt), E, max_m, N, K, _p(out)))
        return out


def load(threads: int = 1) -> COracle:
    """The C oracle, built first when its library is missing or older than its source."""
    from . import build_ref
    src_time = max(os.path.getmtime(build_ref.SRC),
                   os.path.getmtime(os.path.join(HERE, "moe_ref.h")))
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < src_time:
        build_ref.build()
    return COracle(LIB_PATH, threads)
