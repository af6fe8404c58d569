"""Python front of the CPU oracle (``liboracle.so``, built from moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. Nothing here touches
the HIP library; the two share no code.

A layer is described by any object with the attributes of
``moe_synth.Workload`` (T, d, d_ff, E, K, d_shared, latent, act, route,
renormalize, has_rmsnorm, routed_scale, rms_eps); tensors are the host numpy
arrays ``moe_synth.generate`` returns (fp32 arrays, or bf16 as uint16 bits).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ROUTES = {"topk_softmax": 0, "softmax_topk": 1, "sigmoid_bias": 2}
ACTS = {"f32": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only, OpenMP over tokens)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Layer(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int32), ("d_ff", C.c_int32), ("E", C.c_int32),
                ("K", C.c_int32), ("d_shared", C.c_int32), ("latent", C.c_int32),
                ("act", C.c_int32), ("route", C.c_int32), ("renormalize", C.c_int32),
                ("has_rmsnorm", C.c_int32), ("routed_scale", C.c_double),
                ("rms_eps", C.c_double)]


class _Tensors(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "x", "w_router", "bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up",
        "ws_down", "w_lat_down", "w_lat_up", "rms_gamma")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB):
            build(force=True)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.or_route.argtypes = [P, P, P, C.c_int64, P, P, P, P]
        L.or_forward.argtypes = [P, P, P, C.c_int64, P, P, P, P, P]
        L.or_expert_rows.argtypes = [P, P, P, P, P, C.c_int64, P]
        L.or_combine.argtypes = [P, P, P, C.c_int32, P, P, C.c_int64, P]
        L.or_dispatch.argtypes = [C.c_int64, C.c_int32, C.c_int32, P, P, P, P, P, P, P, P]
        L.or_balance_bias.argtypes = [C.c_int32, C.c_int32, C.c_int64, P, C.c_float, P]
        L.or_quantile_balance.argtypes = [P, P, P]
        L.or_router_losses.argtypes = [P, P, P, C.c_double, C.c_double, P]
        L.or_backward.argtypes = [P, P, P, P, C.c_int64, P, C.c_int32] + [P] * 11
        L.or_backward.restype = C.c_int
        for f in ("or_route", "or_forward", "or_expert_rows", "or_combine", "or_dispatch"):
            getattr(L, f).restype = C.c_int
        L.or_silu.argtypes = [C.c_double]
        L.or_silu.restype = C.c_double
        L.or_sigmoid.argtypes = [C.c_double]
        L.or_sigmoid.restype = C.c_double
        L.or_bf16_to_double.argtypes = [C.c_uint16]
        L.or_bf16_to_double.restype = C.c_double
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def silu(x: float) -> float:
    return lib().or_silu(float(x))


def sigmoid(x: float) -> float:
    return lib().or_sigmoid(float(x))


def bf16_to_double(bits: int) -> float:
    return lib().or_bf16_to_double(int(bits))


class Oracle:
    """Per-token fp64 evaluation of one MoE layer on host arrays."""

    def __init__(self, spec, arrays: dict):
        self.spec = spec
        self._keep = {}
        act_np = np.float32 if spec.act == "f32" else np.uint16

        def keep(name, dtype):
            a = arrays.get(name)
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=dtype)
            self._keep[name] = a
            return a.ctypes.data

        self.layer = _Layer(T=spec.T, d=spec.d, d_ff=spec.d_ff, E=spec.E, K=spec.K,
                            d_shared=spec.d_shared, latent=spec.latent, act=ACTS[spec.act],
                            route=ROUTES[spec.route], renormalize=int(spec.renormalize),
                            has_rmsnorm=int(spec.has_rmsnorm),
                            routed_scale=float(spec.routed_scale), rms_eps=float(spec.rms_eps))
        self.tensors = _Tensors(
            x=keep("x", act_np), w_router=keep("w_router", np.float32),
            bias=keep("bias", np.float32), w_gate=keep("w_gate", act_np),
            w_up=keep("w_up", act_np), w_down=keep("w_down", act_np),
            ws_gate=keep("ws_gate", act_np), ws_up=keep("ws_up", act_np),
            ws_down=keep("ws_down", act_np), w_lat_down=keep("w_lat_down", act_np),
            w_lat_up=keep("w_lat_up", act_np), rms_gamma=keep("rms_gamma", np.float32))
        if spec.d_shared and self.tensors.ws_gate is None:
            raise ValueError("layer has shared experts but no shared weights were given")

    def _tokens(self, tokens):
        if tokens is None:
            return None, self.spec.T
        t = np.ascontiguousarray(tokens, dtype=np.int64)
        return t, len(t)

    def route(self, tokens=None):
        """(idx [n,K] int32, g [n,K] f64, gap [n] f64, top [n,K+1] f64)."""
        t, n = self._tokens(tokens)
        K = self.spec.K
        idx = np.empty((n, K), np.int32)
        g = np.empty((n, K), np.float64)
        gap = np.empty(n, np.float64)
        top = np.empty((n, K + 1), np.float64)
        _check(lib().or_route(C.byref(self.layer), C.byref(self.tensors), _p(t), n,
                              _p(idx), _p(g), _p(gap), _p(top)), "route")
        return idx, g, gap, top

    def forward(self, tokens=None, idx_override=None):
        """(out [n,d] f64, idx, g, gap) for the listed tokens (all if None)."""
        t, n = self._tokens(tokens)
        K = self.spec.K
        ov = None if idx_override is None else np.ascontiguousarray(idx_override, np.int32)
        out = np.empty((n, self.spec.d), np.float64)
        idx = np.empty((n, K), np.int32)
        g = np.empty((n, K), np.float64)
        gap = np.empty(n, np.float64)
        _check(lib().or_forward(C.byref(self.layer), C.byref(self.tensors), _p(t), n,
                                _p(ov), _p(out), _p(idx), _p(g), _p(gap)), "forward")
        return out, idx, g, gap

    def quantile_balance(self):
        """QuantileBalancer update over all T tokens (sigmoid routing): the new
        centred bias [E] in fp64."""
        out = np.zeros(self.spec.E, dtype=np.float64)
        _check(lib().or_quantile_balance(C.byref(self.layer), C.byref(self.tensors), _p(out)),
               "or_quantile_balance")
        return out

    def router_losses(self, counts, alpha: float, z_weight: float):
        """(load-balancing loss, router z-loss) over all T tokens, fp64."""
        c = np.ascontiguousarray(counts, dtype=np.int32)
        out = np.zeros(2, dtype=np.float64)
        _check(lib().or_router_losses(C.byref(self.layer), C.byref(self.tensors), _p(c),
                                      float(alpha), float(z_weight), _p(out)), "or_router_losses")
        return float(out[0]), float(out[1])

    def backward(self, d_out, tokens=None, idx_override=None, experts="all",
                 router=True, shared=True, latent=True):
        """Backward of the layer in fp64 for output gradients
        d_out [n, d] of the listed tokens (all if None). Returns a dict: dx
        [n, d]; w_router [E, d] (router=True); w_gate / w_up [E or 1, d_ff, d]
        and w_down [E or 1, d, d_ff] for experts="all", one expert id, or None;
        ws_gate / ws_up [d_shared, d], ws_down [d, d_shared] (shared=True);
        latent layers: w_lat_down [L, d], w_lat_up [d, L], rms_gamma [L]
        (latent=True; expert gradients then at width L). Weight gradients are
        summed over the listed tokens only."""
        sp = self.spec
        t, n = self._tokens(tokens)
        dy = np.ascontiguousarray(d_out, np.float64)
        assert dy.shape == (n, sp.d)
        ov = None if idx_override is None else np.ascontiguousarray(idx_override, np.int32)
        want = -1 if experts == "all" else (-2 if experts is None else int(experts))
        ne = sp.E if want == -1 else 1
        out = {"dx": np.empty((n, sp.d))}
        if router:
            out["w_router"] = np.empty((sp.E, sp.d))
        de = sp.latent or sp.d
        if want >= -1:
            out["w_gate"] = np.empty((ne, sp.d_ff, de))
            out["w_up"] = np.empty((ne, sp.d_ff, de))
            out["w_down"] = np.empty((ne, de, sp.d_ff))
        if shared and sp.d_shared:
            out["ws_gate"] = np.empty((sp.d_shared, sp.d))
            out["ws_up"] = np.empty((sp.d_shared, sp.d))
            out["ws_down"] = np.empty((sp.d, sp.d_shared))
        if latent and sp.latent:
            out["w_lat_down"] = np.empty((sp.latent, sp.d))
            out["w_lat_up"] = np.empty((sp.d, sp.latent))
            if sp.has_rmsnorm:
                out["rms_gamma"] = np.empty(sp.latent)
        g = out.get
        _check(lib().or_backward(C.byref(self.layer), C.byref(self.tensors), _p(dy), _p(t), n,
                                 _p(ov), want, _p(g("dx")), _p(g("w_router")), _p(g("w_gate")),
                                 _p(g("w_up")), _p(g("w_down")), _p(g("ws_gate")),
                                 _p(g("ws_up")), _p(g("ws_down")), _p(g("w_lat_down")),
                                 _p(g("w_lat_up")), _p(g("rms_gamma"))), "or_backward")
        return out

    def expert_rows(self, rows, expert, scale=None):
        """fp64 scale[p] * FFN_{expert[p]}(rows[p]) at the routed width."""
        act_np = np.float32 if self.spec.act == "f32" else np.uint16
        rows = np.ascontiguousarray(rows, act_np)
        expert = np.ascontiguousarray(expert, np.int32)
        sc = None if scale is None else np.ascontiguousarray(scale, np.float32)
        n = len(expert)
        de = self.spec.latent or self.spec.d
        out = np.empty((n, de), np.float64)
        _check(lib().or_expert_rows(C.byref(self.layer), C.byref(self.tensors), _p(rows),
                                    _p(expert), _p(sc), n, _p(out)), "expert_rows")
        return out

    def combine(self, y_rows, inv, tokens=None):
        """fp64 shared(x_t) + routed combine of y_rows through inv."""
        y_dtype = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1,
                   np.dtype(np.float64): 2}[y_rows.dtype]
        y_rows = np.ascontiguousarray(y_rows)
        inv = np.ascontiguousarray(inv, np.int32)
        t, n = self._tokens(tokens)
        out = np.empty((n, self.spec.d), np.float64)
        _check(lib().or_combine(C.byref(self.layer), C.byref(self.tensors), _p(y_rows),
                                y_dtype, _p(inv), _p(t), n, _p(out)), "combine")
        return out


def dispatch(idx, g, E: int) -> dict:
    """Stable counting sort of the flattened assignments by expert id."""
    idx = np.ascontiguousarray(idx, np.int32)
    T, K = idx.shape
    gf = None if g is None else np.ascontiguousarray(g, np.float32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    st = np.empty(T * K, np.int32)
    inv = np.empty(T * K, np.int32)
    sw = np.empty(T * K, np.float32)
    _check(lib().or_dispatch(T, K, E, _p(idx), _p(gf), _p(counts), _p(offsets), _p(perm),
                             _p(st), _p(inv), _p(sw) if gf is not None else None), "dispatch")
    return dict(counts=counts, offsets=offsets, perm=perm, sorted_token=st, inv=inv,
                sorted_w=sw if gf is not None else None)


def balance_bias(counts, bias, alpha: float, n_tokens: int, K: int) -> np.ndarray:
    """Bias-based balancer step (Part 3, section 14.3): returns the new fp32
    bias for per-expert counts of a step with n_tokens tokens and top-K."""
    c = np.ascontiguousarray(counts, dtype=np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    assert c.shape == b.shape and c.ndim == 1
    _check(lib().or_balance_bias(len(c), K, n_tokens, _p(c), alpha, _p(b)), "or_balance_bias")
    return b
