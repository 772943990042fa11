"""ctypes binding of libmoe.so (include/moe.h), with the same entry-point names.

Argument marshalling only: torch tensors are passed as device pointers with the current
HIP stream, outputs the caller omits are allocated with torch.empty, and a non-zero
status raises MoeError. Every step of the computation runs in libmoe.so; there is no
other code path, and a missing library raises at the first call.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_OVERLAP, MOE_ERR_WORKSPACE, \
    MOE_ERR_LAUNCH = range(6)
DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
TORCH_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
TORCH_OF = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}
SCORING = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2}
LAYOUTS = {"stacked": 0, "interleaved": 1}
BACKENDS = {"auto": 0, "staged": 1, "indexed": 2}
ABI_VERSION = 2
# name -> (layout, alpha, beta, limit, kind); the constants swigluoai fixes; kind 1 is
# gelu_and_mul (stacked rows, no constants).
ACTIVATIONS = {"silu_and_mul": (0, 1.0, 0.0, 0.0, 0), "swigluoai": (1, 1.702, 1.0, 7.0, 0),
               "gelu_and_mul": (0, 0.0, 0.0, 0.0, 1)}

# Every symbol include/moe.h declares.
SYMBOLS = ("moe_status_str", "moe_abi_version", "moe_route", "moe_permute_workspace_size",
           "moe_permute",
           "moe_grouped_gemm_swiglu", "moe_grouped_gemm", "moe_combine",
           "moe_ffn_workspace_size", "moe_ffn_backend", "moe_ffn_forward",
           "moe_grouped_gemm_fp8_masked", "moe_swiglu", "moe_grouped_gemm_layout_workspace_size",
           "moe_grouped_gemm_layout", "moe_layout_workspace_size", "moe_permute_align",
           "moe_pre_permute", "moe_ffn_forward_noalloc")
# moe_ffn_forward_noalloc's fixed scratch (MOE_FFN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeRouteCfg(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("num_expert_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("local_expert_start", ctypes.c_int32), ("local_expert_count", ctypes.c_int32),
                ("router_probs_dtype", ctypes.c_int32), ("logits_dtype", ctypes.c_int32)]


class MoeActCfg(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("beta", ctypes.c_float), ("limit", ctypes.c_float), ("kind", ctypes.c_int32)]


class MoeFfnCfg(ctypes.Structure):
    _fields_ = [("route", MoeRouteCfg), ("act", MoeActCfg), ("T", ctypes.c_int64),
                ("H", ctypes.c_int64), ("E", ctypes.c_int64), ("F", ctypes.c_int64),
                ("F_shared", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("backend", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib().moe_status_str(status).decode()} (status {status})")


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def lib():
    """Load libmoe.so once and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "python -m mixture_experts_ffn_moerouter_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_abi_version.restype = ctypes.c_int
        L.moe_abi_version.argtypes = []
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.moe_abi_version()}, this "
                               f"binding needs {ABI_VERSION}; rebuild the library")
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [_P, _I64, _I64, _P, _P, ctypes.POINTER(MoeRouteCfg), _P, _P,
                                _P, _P, _P]
        L.moe_permute_workspace_size.restype = ctypes.c_size_t
        L.moe_permute_workspace_size.argtypes = [_I64, _I64, _I64]
        L.moe_permute.restype = ctypes.c_int
        L.moe_permute.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P, _I64, _I32, _P, _P,
                                  ctypes.c_size_t, _P]
        L.moe_grouped_gemm_swiglu.restype = ctypes.c_int
        L.moe_grouped_gemm_swiglu.argtypes = [_P, _P, _I32, _I64, _I64, _P, _P, _I64, _I64,
                                              _P, _I32, ctypes.POINTER(MoeActCfg), _P, _P]
        L.moe_grouped_gemm.restype = ctypes.c_int
        L.moe_grouped_gemm.argtypes = [_P, _P, _I32, _I64, _I64, _P, _P, _I64, _I64, _P,
                                       _I32, _I32, _P, _P]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [_P, _I32, _I64, _P, _P, _I64, _I64, _I64, ctypes.c_float,
                                  _P, _I32, _P]
        L.moe_grouped_gemm_layout_workspace_size.restype = ctypes.c_size_t
        L.moe_grouped_gemm_layout_workspace_size.argtypes = [_I64]
        L.moe_grouped_gemm_layout.restype = ctypes.c_int
        L.moe_grouped_gemm_layout.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I64, _I32, _P,
                                              _I64, ctypes.POINTER(MoeActCfg), _I32, _I32, _P,
                                              _P, ctypes.c_size_t, _P]
        L.moe_layout_workspace_size.restype = ctypes.c_size_t
        L.moe_layout_workspace_size.argtypes = [_I64, _I64, _I64, _I64]
        L.moe_permute_align.restype = ctypes.c_int
        L.moe_permute_align.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]
        L.moe_pre_permute.restype = ctypes.c_int
        L.moe_pre_permute.argtypes = [_P, _I64, _I64, _I32, _P, _I64, _I64, _I32, _I64, _I64,
                                      _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_ffn_workspace_size.restype = ctypes.c_size_t
        L.moe_ffn_workspace_size.argtypes = [ctypes.POINTER(MoeFfnCfg)]
        L.moe_ffn_backend.restype = ctypes.c_int
        L.moe_ffn_backend.argtypes = [ctypes.POINTER(MoeFfnCfg), ctypes.c_int]
        L.moe_grouped_gemm_fp8_masked.restype = ctypes.c_int
        L.moe_grouped_gemm_fp8_masked.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                                  _P, _P]
        L.moe_swiglu.restype = ctypes.c_int
        L.moe_swiglu.argtypes = [_P, _P, _I64, _I64, _I32, _I32, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_float, _P, _P]
        L.moe_ffn_forward.restype = ctypes.c_int
        L.moe_ffn_forward.argtypes = [ctypes.POINTER(MoeFfnCfg)] + [_P] * 15 + \
            [ctypes.c_size_t, _P]
        L.moe_ffn_forward_noalloc.restype = ctypes.c_int
        L.moe_ffn_forward_noalloc.argtypes = [ctypes.POINTER(MoeFfnCfg)] + [_P] * 15
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ----------------------------------------------------------------------- configs
def route_cfg(top_k: int, scoring: str = "softmax", renormalize: bool = False,
              routed_scaling_factor: float = 1.0, num_expert_group: int = 1,
              topk_group: int = 1, local_expert_start: int = 0, local_expert_count: int = 0,
              router_probs_dtype: str = "f32") -> MoeRouteCfg:
    return MoeRouteCfg(top_k, SCORING[scoring], int(bool(renormalize)),
                       float(routed_scaling_factor), num_expert_group, topk_group,
                       local_expert_start, local_expert_count, DTYPES[router_probs_dtype])


def act_cfg(act) -> MoeActCfg:
    """'silu_and_mul', 'swigluoai', 'gelu_and_mul', or a (layout, alpha, beta, limit[,
    kind]) tuple."""
    if isinstance(act, str):
        return MoeActCfg(*ACTIVATIONS[act])
    layout, alpha, beta, limit = act[:4]
    kind = act[4] if len(act) > 4 else 0
    return MoeActCfg(LAYOUTS[layout] if isinstance(layout, str) else layout, alpha, beta, limit,
                     kind)


def ffn_cfg(cfg, backend: str = "auto") -> MoeFfnCfg:
    """From a mixture_experts_ffn_moerouter_amd.inputs.MoEConfig."""
    rc = route_cfg(cfg.K, cfg.scoring, cfg.renormalize, cfg.rsf, cfg.G, cfg.TG)
    return MoeFfnCfg(rc, act_cfg(cfg.act), cfg.T, cfg.H, cfg.E, cfg.F, cfg.F_s,
                     DTYPES[cfg.dtype], BACKENDS[backend])


# ----------------------------------------------------------------------- entry points
def moe_route(logits, cfg: MoeRouteCfg, correction_bias=None, expert_ids=None,
              topk_weights=None, topk_ids=None, router_probs=None, weight_scale=None,
              with_router_probs: bool = False, stream=None):
    T, E = logits.shape
    K = cfg.top_k
    dev = logits.device
    cfg = MoeRouteCfg.from_buffer_copy(cfg)
    cfg.logits_dtype = TORCH_DTYPES[logits.dtype]
    topk_weights = torch.empty((T, K), dtype=torch.float32, device=dev) \
        if topk_weights is None else topk_weights
    topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev) if topk_ids is None \
        else topk_ids
    if with_router_probs and router_probs is None:
        dt = TORCH_OF[cfg.router_probs_dtype]
        router_probs = torch.empty((T, cfg.local_expert_count), dtype=dt, device=dev)
        weight_scale = torch.empty((T,), dtype=dt, device=dev)
    _check("moe_route", lib().moe_route(
        _ptr(logits), T, E, _ptr(correction_bias), _ptr(expert_ids), ctypes.byref(cfg),
        _ptr(topk_weights), _ptr(topk_ids), _ptr(router_probs), _ptr(weight_scale),
        _stream(stream)))
    return topk_weights, topk_ids, router_probs, weight_scale


def moe_permute_workspace_size(T: int, K: int, E: int) -> int:
    return lib().moe_permute_workspace_size(T, K, E)


def moe_permute(topk_ids, num_experts: int, hidden=None, expert_offsets=None,
                sorted_route=None, route_pos=None, permuted=None, workspace=None,
                stream=None):
    T, K = topk_ids.shape
    R = T * K
    dev = topk_ids.device
    expert_offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev) \
        if expert_offsets is None else expert_offsets
    sorted_route = torch.empty(R, dtype=torch.int32, device=dev) if sorted_route is None \
        else sorted_route
    route_pos = torch.empty(R, dtype=torch.int32, device=dev) if route_pos is None \
        else route_pos
    H, dt = 0, 0
    if hidden is not None:
        H = hidden.shape[1]
        dt = TORCH_DTYPES[hidden.dtype]
        permuted = torch.empty((R, H), dtype=hidden.dtype, device=dev) if permuted is None \
            else permuted
    if workspace is None:
        workspace = torch.empty(max(1, moe_permute_workspace_size(T, K, num_experts)),
                                dtype=torch.uint8, device=dev)
    _check("moe_permute", lib().moe_permute(
        _ptr(topk_ids), T, K, num_experts, _ptr(expert_offsets), _ptr(sorted_route),
        _ptr(route_pos), _ptr(hidden), H, dt, _ptr(permuted), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return expert_offsets, sorted_route, route_pos, permuted


def moe_grouped_gemm_swiglu(a, w_gate_up, expert_offsets, act="silu_and_mul",
                            b_gate_up=None, a_rows=None, a_rows_div: int = 1, M=None,
                            out=None, stream=None):
    E, twoF, H = w_gate_up.shape
    F = twoF // 2
    M = (a.shape[0] if a_rows is None else a_rows.shape[0]) if M is None else M
    out = torch.empty((M, F), dtype=a.dtype, device=a.device) if out is None else out
    ac = act_cfg(act)
    _check("moe_grouped_gemm_swiglu", lib().moe_grouped_gemm_swiglu(
        _ptr(a), _ptr(a_rows), a_rows_div, M, H, _ptr(w_gate_up), _ptr(b_gate_up), E, F,
        _ptr(expert_offsets), TORCH_DTYPES[a.dtype], ctypes.byref(ac), _ptr(out),
        _stream(stream)))
    return out


def moe_grouped_gemm(a, b, expert_offsets, bias=None, out_dtype=None, a_rows=None,
                     a_rows_div: int = 1, M=None, out=None, stream=None):
    E, N, K = b.shape
    M = (a.shape[0] if a_rows is None else a_rows.shape[0]) if M is None else M
    out_dtype = a.dtype if out_dtype is None else out_dtype
    out = torch.empty((M, N), dtype=out_dtype, device=a.device) if out is None else out
    _check("moe_grouped_gemm", lib().moe_grouped_gemm(
        _ptr(a), _ptr(a_rows), a_rows_div, M, K, _ptr(b), _ptr(bias), E, N,
        _ptr(expert_offsets), TORCH_DTYPES[a.dtype], TORCH_DTYPES[out_dtype], _ptr(out),
        _stream(stream)))
    return out


def moe_combine(y, topk_weights, route_pos, scale: float = 1.0, out_dtype=None, out=None,
                stream=None):
    """y: [rows, H] expert outputs, or a masked [E, max_m, H] slab; route_pos: the row of
    each route (negative: no contribution)."""
    T, K = topk_weights.shape
    H = y.shape[-1]
    out_dtype = y.dtype if out_dtype is None else out_dtype
    out = torch.empty((T, H), dtype=out_dtype, device=y.device) if out is None else out
    _check("moe_combine", lib().moe_combine(
        _ptr(y), TORCH_DTYPES[y.dtype], y.numel() // max(H, 1), _ptr(topk_weights),
        _ptr(route_pos), T, K, H, float(scale), _ptr(out), TORCH_DTYPES[out_dtype],
        _stream(stream)))
    return out


LAYOUT_KINDS = {"contiguous": 0, "per_row": 1, "masked": 2}


def moe_layout_workspace_size(T: int, K: int, E: int, block_size: int = 1) -> int:
    return lib().moe_layout_workspace_size(T, K, E, block_size)


def moe_permute_align(topk_ids, num_experts: int, block_size: int = 64, workspace=None,
                      stream=None):
    """[TO] MoEPermuteAlignFwdOp: (sorted_token_ids, expert_ids, num_tokens_post_pad)."""
    T, K = topk_ids.shape
    E, bs = num_experts, block_size
    length = T * K + (E + 1) * (bs - 1)
    dev = topk_ids.device
    sorted_ids = torch.empty(length, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(-(-length // bs), dtype=torch.int32, device=dev)
    num = torch.empty(1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(1, moe_layout_workspace_size(T, K, E, bs)),
                                dtype=torch.uint8, device=dev)
    _check("moe_permute_align", lib().moe_permute_align(
        _ptr(topk_ids), T, K, E, bs, _ptr(sorted_ids), _ptr(expert_ids), _ptr(num),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return sorted_ids, expert_ids, num


def moe_pre_permute(hidden, topk_ids, num_experts: int, layout: str = "contiguous",
                    block_size: int = 1, max_m: int = 0, workspace=None, stream=None):
    """[TO] MoEPrePermuteFwdOp: (expert_input, layout_metadata, inverse_indices)."""
    T, H = hidden.shape
    K = topk_ids.shape[1]
    E = num_experts
    dev = hidden.device
    bs = 1 if layout == "masked" else block_size
    if layout == "masked":
        expert_input = torch.empty((E, max_m, H), dtype=hidden.dtype, device=dev)
        meta = torch.empty(E, dtype=torch.int32, device=dev)
    else:
        cap = T * K + E * (bs - 1)
        expert_input = torch.empty((cap, H), dtype=hidden.dtype, device=dev)
        meta = torch.empty(cap if layout == "per_row" else E, dtype=torch.int32, device=dev)
    inverse = torch.empty(T * K, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(1, moe_layout_workspace_size(T, K, E, bs)),
                                dtype=torch.uint8, device=dev)
    _check("moe_pre_permute", lib().moe_pre_permute(
        _ptr(hidden), T, H, TORCH_DTYPES[hidden.dtype], _ptr(topk_ids), K, E,
        LAYOUT_KINDS[layout], bs, max_m, _ptr(expert_input), _ptr(meta), _ptr(inverse),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return expert_input, meta, inverse


def moe_grouped_gemm_layout(a, b, layout: str, layout_metadata, bias=None, act=None,
                            out_dtype=None, out=None, workspace=None, stream=None):
    """[TO] MoEGroupedGemmFwdOp over a layout: a [M, K] (contiguous, per_row) or
    [E, max_m, K] (masked); act None (plain) or a gated activation."""
    E, N, K = b.shape
    masked = layout == "masked"
    M = 0 if masked else a.shape[0]
    max_m = a.shape[1] if masked else 0
    Nout = N // 2 if act is not None else N
    out_dtype = a.dtype if out_dtype is None else out_dtype
    if out is None:
        shape = (E, max_m, Nout) if masked else (M, Nout)
        out = torch.empty(shape, dtype=out_dtype, device=a.device)
    if workspace is None and layout == "per_row":
        workspace = torch.empty(lib().moe_grouped_gemm_layout_workspace_size(E),
                                dtype=torch.uint8, device=a.device)
    ac = act_cfg(act) if act is not None else None
    _check("moe_grouped_gemm_layout", lib().moe_grouped_gemm_layout(
        _ptr(a), M, K, _ptr(b), _ptr(bias), E, N, LAYOUT_KINDS[layout], _ptr(layout_metadata),
        max_m, ctypes.byref(ac) if ac is not None else None, TORCH_DTYPES[a.dtype],
        TORCH_DTYPES[out_dtype], _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)))
    return out


def _fp8_bytes(t):
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def moe_grouped_gemm_fp8_masked(a, a_scale, b, b_scale, counts, out=None, stream=None):
    """a [E, max_m, K] and b [E, N, K] as float8_e4m3fn or their uint8 bytes; a_scale
    [E, max_m, K/128] and b_scale [E, N/128, K/128] float32; counts [E] int32. Returns
    out [E, max_m, N] bfloat16 (rows at or past a count are left as they were)."""
    a, b = _fp8_bytes(a), _fp8_bytes(b)
    E, max_m, K = a.shape
    N = b.shape[1]
    out = torch.empty((E, max_m, N), dtype=torch.bfloat16, device=a.device) \
        if out is None else out
    _check("moe_grouped_gemm_fp8_masked", lib().moe_grouped_gemm_fp8_masked(
        _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(counts), E, max_m, K, N,
        _ptr(out), _stream(stream)))
    return out


def moe_swiglu(gate, up=None, alpha: float = 1.0, beta: float = 0.0, limit: float = 0.0,
               fusion: str = "stacked", out=None, stream=None):
    """[MR] SwiGLU: gate and up [.., F], or gate [.., 2F] holding both halves (fusion
    'stacked' = gate then up, 'interleaved'). Returns out [.., F] in gate's dtype."""
    F = gate.shape[-1] if up is not None else gate.shape[-1] // 2
    rows = gate.numel() // max(1, gate.shape[-1])
    out = torch.empty((*gate.shape[:-1], F), dtype=gate.dtype, device=gate.device) \
        if out is None else out
    _check("moe_swiglu", lib().moe_swiglu(
        _ptr(gate), _ptr(up), rows, F, TORCH_DTYPES[gate.dtype], LAYOUTS[fusion],
        float(alpha), float(beta), float(limit), _ptr(out), _stream(stream)))
    return out


def moe_ffn_workspace_size(cfg: MoeFfnCfg) -> int:
    return lib().moe_ffn_workspace_size(ctypes.byref(cfg))


def moe_ffn_backend(cfg: MoeFfnCfg, has_bias: bool = False) -> int:
    return lib().moe_ffn_backend(ctypes.byref(cfg), int(bool(has_bias)))


def moe_ffn_forward(cfg: MoeFfnCfg, hidden, logits, w_gate_up, w_down, correction_bias=None,
                    expert_ids=None, b_gate_up=None, b_down=None, shared_w_gate_up=None,
                    shared_w_down=None, out=None, shared_out=None, topk_weights_out=None,
                    topk_ids_out=None, workspace=None, stream=None):
    """Returns (out, shared_out or None)."""
    T, H = hidden.shape
    dev = hidden.device
    cfg = MoeFfnCfg.from_buffer_copy(cfg)
    cfg.route.logits_dtype = TORCH_DTYPES[logits.dtype]
    out = torch.empty((T, H), dtype=hidden.dtype, device=dev) if out is None else out
    if cfg.F_shared > 0 and shared_out is None:
        shared_out = torch.empty((T, H), dtype=hidden.dtype, device=dev)
    if workspace is None:
        workspace = torch.empty(max(1, moe_ffn_workspace_size(cfg)), dtype=torch.uint8,
                                device=dev)
    _check("moe_ffn_forward", lib().moe_ffn_forward(
        ctypes.byref(cfg), _ptr(hidden), _ptr(logits), _ptr(correction_bias),
        _ptr(expert_ids), _ptr(w_gate_up), _ptr(w_down), _ptr(b_gate_up), _ptr(b_down),
        _ptr(shared_w_gate_up), _ptr(shared_w_down), _ptr(out), _ptr(shared_out),
        _ptr(topk_weights_out), _ptr(topk_ids_out), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out, shared_out


def moe_ffn_forward_noalloc(cfg: MoeFfnCfg, hidden, logits, w_gate_up, w_down,
                            correction_bias=None, expert_ids=None, b_gate_up=None, b_down=None,
                            shared_w_gate_up=None, shared_w_down=None, out=None,
                            shared_out=None, topk_weights_out=None, topk_ids_out=None,
                            stream=None):
    """moe_ffn_forward on the library's fixed scratch (no workspace argument; the library
    allocates nothing). Outputs the caller omits are still allocated here by torch."""
    T, H = hidden.shape
    dev = hidden.device
    cfg = MoeFfnCfg.from_buffer_copy(cfg)
    cfg.route.logits_dtype = TORCH_DTYPES[logits.dtype]
    out = torch.empty((T, H), dtype=hidden.dtype, device=dev) if out is None else out
    if cfg.F_shared > 0 and shared_out is None:
        shared_out = torch.empty((T, H), dtype=hidden.dtype, device=dev)
    _check("moe_ffn_forward_noalloc", lib().moe_ffn_forward_noalloc(
        ctypes.byref(cfg), _ptr(hidden), _ptr(logits), _ptr(correction_bias),
        _ptr(expert_ids), _ptr(w_gate_up), _ptr(w_down), _ptr(b_gate_up), _ptr(b_down),
        _ptr(shared_w_gate_up), _ptr(shared_w_down), _ptr(out), _ptr(shared_out),
        _ptr(topk_weights_out), _ptr(topk_ids_out), _stream(stream)))
    return out, shared_out
