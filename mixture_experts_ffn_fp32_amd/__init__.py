"""Python binding of libmoe.so, the MI355X MoE SwiGLU feed-forward library.

Argument marshalling only: every function below forwards device pointers
(``tensor.data_ptr()``) and the current HIP stream to the C entry point of the
same name declared in include/moe.h. No step of the layer runs in Python, and
there is no fallback: if libmoe.so is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

EXPORTS = ("moe_strerror", "moe_stage_name", "moe_workspace_size", "moe_route", "moe_dispatch",
           "moe_expert_ffn", "moe_combine", "moe_forward", "moe_quantile_balance",
           "moe_balance_bias", "moe_router_losses", "moe_plan", "moe_backward_workspace_size",
           "moe_backward", "moe_peak", "moe_forward_noalloc")

MOE_F32, MOE_BF16 = 0, 1
ROUTE_MODES = {"topk_softmax": 0, "softmax_topk": 1, "sigmoid_bias": 2}
STAGES = {"route": 0, "dispatch": 1, "latent_down": 2, "expert_gate_up": 3, "expert_down": 4,
          "shared_gate_up": 5, "combine": 6}
TIE_EPS = 1e-5


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


class MoeDesc(C.Structure):
    _fields_ = [("T", C.c_int64), ("d_model", C.c_int32), ("d_ff", C.c_int32),
                ("n_experts", C.c_int32), ("top_k", C.c_int32), ("d_shared", C.c_int32),
                ("latent", C.c_int32), ("act_dtype", C.c_int32), ("route_mode", C.c_int32),
                ("renormalize", C.c_int32), ("has_rmsnorm", C.c_int32),
                ("routed_scale", C.c_float), ("rms_eps", C.c_float)]


class MoeWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "w_router", "bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
        "w_lat_down", "w_lat_up", "rms_gamma")]


class MoePlanInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "merged_shared", "gate_up_pipelined", "gate_up_tile_m", "gate_up_tile_n",
        "down_pipelined", "down_tile_m", "down_tile_n", "router_per_token",
        "dispatch_one_workgroup", "backward_in_place", "persistent")]


class MoeGrads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down", "w_lat_down",
        "w_lat_up", "rms_gamma")]


class MoeProbe(C.Structure):
    _fields_ = [("stage", C.c_int32), ("repeat", C.c_int32), ("ev_begin", C.c_void_p),
                ("ev_end", C.c_void_p)]


_lib = None


def lib():
    """Load libmoe.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        P, S = C.c_void_p, C.c_size_t
        L.moe_strerror.argtypes = [C.c_int]
        L.moe_strerror.restype = C.c_char_p
        L.moe_stage_name.argtypes = [C.c_int]
        L.moe_stage_name.restype = C.c_char_p
        L.moe_workspace_size.argtypes = [P, C.POINTER(C.c_size_t)]
        L.moe_route.argtypes = [P, P, P, P, P, P, P, P, S, P]
        L.moe_dispatch.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.moe_expert_ffn.argtypes = [P, P, P, P, P, P, P, P, S, P]
        L.moe_combine.argtypes = [P, P, P, P, P, P, P, S, P]
        L.moe_forward.argtypes = [P, P, P, P, P, P, P, S, P, P]
        L.moe_balance_bias.argtypes = [C.c_int32, C.c_int32, C.c_int64, P, C.c_float, P, P]
        L.moe_quantile_balance.argtypes = [P, P, P, P, P, S, P]
        L.moe_router_losses.argtypes = [P, P, P, P, C.c_float, C.c_float, P, P, S, P]
        L.moe_plan.argtypes = [P, P]
        L.moe_backward_workspace_size.argtypes = [P, C.POINTER(C.c_size_t)]
        L.moe_backward.argtypes = [P, P, P, P, P, P, P, S, P]
        L.moe_peak.argtypes = [C.c_int32] * 4 + [P, P, P]
        L.moe_forward_noalloc.argtypes = [P, P, P, P, P, P, P]
        for f in ("moe_workspace_size", "moe_route", "moe_dispatch", "moe_expert_ffn",
                  "moe_combine", "moe_forward", "moe_balance_bias", "moe_quantile_balance",
                  "moe_router_losses", "moe_plan", "moe_backward_workspace_size",
                  "moe_backward", "moe_peak", "moe_forward_noalloc"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def stage_name(stage: int) -> str:
    return lib().moe_stage_name(int(stage)).decode()


def _ptr(t):
    """Device address of a tensor for an array argument of the C ABI (all of
    them are device memory); None is the null pointer. Host tensors and
    non-contiguous views are refused here, before anything is launched."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"libmoe takes device tensors; got a host tensor {tuple(t.shape)} "
                         f"{t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"libmoe takes contiguous tensors; got a strided view "
                         f"{tuple(t.shape)} {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ok(rc: int, what: str):
    if rc != 0:
        raise MoeError(rc, what)


def make_desc(spec) -> MoeDesc:
    """moe_desc of a layer described like ``moe_synth.Workload``."""
    return MoeDesc(T=spec.T, d_model=spec.d, d_ff=spec.d_ff, n_experts=spec.E, top_k=spec.K,
                   d_shared=spec.d_shared, latent=spec.latent,
                   act_dtype=MOE_BF16 if spec.act == "bf16" else MOE_F32,
                   route_mode=ROUTE_MODES[spec.route], renormalize=int(spec.renormalize),
                   has_rmsnorm=int(spec.has_rmsnorm), routed_scale=float(spec.routed_scale),
                   rms_eps=float(spec.rms_eps))


def make_weights(t: dict) -> MoeWeights:
    """moe_weights from a dict of device tensors (keys as in moe_weights).
    The caller keeps the tensors alive while the struct is in use."""
    return MoeWeights(**{k: _ptr(t.get(k)) for k, _ in MoeWeights._fields_})


def moe_plan(desc: MoeDesc) -> dict:
    """How moe_forward runs this layer (kernel paths and tile shapes)."""
    info = MoePlanInfo()
    _ok(lib().moe_plan(C.byref(desc), C.byref(info)), "moe_plan")
    return {n: int(getattr(info, n)) for n, _ in MoePlanInfo._fields_}


def moe_backward_workspace_size(desc: MoeDesc) -> int:
    n = C.c_size_t(0)
    _ok(lib().moe_backward_workspace_size(C.byref(desc), C.byref(n)),
        "moe_backward_workspace_size")
    return n.value


def moe_backward(desc, weights, x, d_out, d_x, grads: dict, ws, stream=None):
    """Backward of the layer: d_x (act dtype) and fp32 weight gradients into
    the device tensors of `grads` (keys as MoeGrads; missing keys are not
    computed)."""
    g = MoeGrads(**{k: _ptr(grads.get(k)) for k, _ in MoeGrads._fields_})
    _ok(lib().moe_backward(C.byref(desc), C.byref(weights), _ptr(x), _ptr(d_out), _ptr(d_x),
                           C.byref(g), _ptr(ws), _nbytes(ws), _stream(stream)), "moe_backward")


def moe_workspace_size(desc: MoeDesc) -> int:
    n = C.c_size_t(0)
    _ok(lib().moe_workspace_size(C.byref(desc), C.byref(n)), "moe_workspace_size")
    return n.value


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_route(desc, weights, x, idx, g, gap=None, top_scores=None, ws=None, stream=None):
    _ok(lib().moe_route(C.byref(desc), C.byref(weights), _ptr(x), _ptr(idx), _ptr(g), _ptr(gap),
                        _ptr(top_scores), _ptr(ws), _nbytes(ws), _stream(stream)), "moe_route")


def moe_quantile_balance(desc, weights, x, new_bias, ws, stream=None):
    """QuantileBalancer update of a sigmoid-routed layer: new_bias fp32 [E]."""
    _ok(lib().moe_quantile_balance(C.byref(desc), C.byref(weights), _ptr(x), _ptr(new_bias),
                                   _ptr(ws), _nbytes(ws), _stream(stream)), "moe_quantile_balance")


def moe_router_losses(desc, weights, x, counts, alpha, z_weight, losses, ws, stream=None):
    """Load-balancing loss and router z-loss of one step into losses fp32 [2]
    (counts: int32 [E] loads of the same tokens)."""
    _ok(lib().moe_router_losses(C.byref(desc), C.byref(weights), _ptr(x), _ptr(counts),
                                float(alpha), float(z_weight), _ptr(losses), _ptr(ws),
                                _nbytes(ws), _stream(stream)), "moe_router_losses")


def moe_balance_bias(n_experts, top_k, n_tokens, counts, alpha, bias, stream=None):
    """One bias-based balancer step on device arrays (counts int32 [E], bias
    fp32 [E], updated in place)."""
    _ok(lib().moe_balance_bias(int(n_experts), int(top_k), int(n_tokens), _ptr(counts),
                               float(alpha), _ptr(bias), _stream(stream)), "moe_balance_bias")


def moe_dispatch(desc, idx, g, rows, counts, offsets, perm, sorted_token, inv, sorted_w,
                 rows_sorted, ws, stream=None):
    _ok(lib().moe_dispatch(C.byref(desc), _ptr(idx), _ptr(g), _ptr(rows), _ptr(counts),
                           _ptr(offsets), _ptr(perm), _ptr(sorted_token), _ptr(inv),
                           _ptr(sorted_w), _ptr(rows_sorted), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
        "moe_dispatch")


def moe_expert_ffn(desc, weights, rows, row_index, offsets, row_scale, y_sorted, ws, stream=None):
    _ok(lib().moe_expert_ffn(C.byref(desc), C.byref(weights), _ptr(rows), _ptr(row_index),
                             _ptr(offsets), _ptr(row_scale), _ptr(y_sorted), _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(),
                             _stream(stream)), "moe_expert_ffn")


def moe_combine(desc, weights, x, y_sorted, inv, out, ws, stream=None):
    _ok(lib().moe_combine(C.byref(desc), C.byref(weights), _ptr(x), _ptr(y_sorted), _ptr(inv),
                          _ptr(out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                          _stream(stream)), "moe_combine")


def moe_forward(desc, weights, x, out, counts=None, n_near_ties=None, ws=None, probe=None,
                stream=None):
    _ok(lib().moe_forward(C.byref(desc), C.byref(weights), _ptr(x), _ptr(out), _ptr(counts),
                          _ptr(n_near_ties), _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(),
                          None if probe is None else C.byref(probe), _stream(stream)),
        "moe_forward")


def moe_peak(mode, threads, groups, iters, clk, sink, stream=None):
    """Peak-rate microbenchmark launch (measurement helper; see include/moe.h)."""
    _ok(lib().moe_peak(int(mode), int(threads), int(groups), int(iters), _ptr(clk), _ptr(sink),
                       _stream(stream)), "moe_peak")


def moe_forward_noalloc(desc, weights, x, out, counts=None, n_near_ties=None, stream=None):
    """moe_forward in the library's static device scratch (allocates nothing)."""
    _ok(lib().moe_forward_noalloc(C.byref(desc), C.byref(weights), _ptr(x), _ptr(out),
                                  _ptr(counts), _ptr(n_near_ties), _stream(stream)),
        "moe_forward_noalloc")


SCRATCH_BYTES = 64 << 20  # MOE_SCRATCH_BYTES


# ----------------------------------------------------------------- plumbing

def to_device(arrays: dict, device="cuda"):
    """Upload host arrays (fp32, or bf16 as uint16 bits) as torch tensors."""
    import numpy as np
    import torch
    out = {}
    for k, v in arrays.items():
        if not isinstance(v, np.ndarray):
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if v.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        out[k] = t.to(device, non_blocking=False)
    return out


class Layer:
    """Device weights + workspace of one layer; forward() calls moe_forward."""

    def __init__(self, spec, dev: dict, device="cuda"):
        import torch
        self.spec = spec
        self.desc = make_desc(spec)
        self.dev = dev
        self.weights = make_weights(dev)
        self.ws = torch.empty(max(1, moe_workspace_size(self.desc)), dtype=torch.uint8,
                              device=device)
        self.act = torch.bfloat16 if spec.act == "bf16" else torch.float32
        self.device = device

    def forward(self, x, out=None, counts=None, n_near_ties=None, probe=None, stream=None):
        import torch
        if out is None:
            out = torch.empty((self.spec.T, self.spec.d), dtype=self.act, device=self.device)
        moe_forward(self.desc, self.weights, x, out, counts, n_near_ties, self.ws, probe, stream)
        return out

    def backward(self, x, d_out, d_x=None, grads=None, stream=None):
        """moe_backward with a workspace of its own (allocated on first use);
        grads: dict of fp32 device tensors to fill (keys as MoeGrads)."""
        import torch
        if getattr(self, "ws_bwd", None) is None:
            self.ws_bwd = torch.empty(max(1, moe_backward_workspace_size(self.desc)),
                                      dtype=torch.uint8, device=self.device)
        if d_x is None:
            d_x = torch.empty((self.spec.T, self.spec.d), dtype=self.act, device=self.device)
        moe_backward(self.desc, self.weights, x, d_out, d_x, grads or {}, self.ws_bwd, stream)
        return d_x
