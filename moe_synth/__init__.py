"""Seeded synthetic inputs for the MoE SwiGLU feed-forward layer.

This module only draws numbers. It holds no step of the method itself (no
routing, no selection, no matmul): it produces the token matrix, router
weights, balance bias and expert / shared / latent weights for the workloads
below, and is the single source of inputs for both the HIP path and the CPU
oracle, which then read identical bytes.

Seeding: ``numpy.random.SeedSequence(1000 + config_no)`` is spawned into a
fixed list of slots (one per tensor family); the expert slot is spawned again
per expert and then per matrix, so any single expert can be regenerated on its
own. Every sample is drawn in fp32 with PCG64; bf16 tensors are the
round-to-nearest-even bf16 of those fp32 samples, stored as ``uint16`` bit
patterns.

Workloads (sizes and distributions as the layer is specified; the pages'
own demos use ``torch.randn`` inputs, so these synthetic draws stand in for
nothing else):

* ``tiny``          T=128 (4x32), d=64, d_ff=128, E=8, K=2, 1 shared, fp32,
                    softmax over all E then top-K then renormalise; no bias;
                    x ~ N(0,1); weights ~ U(+-1/sqrt(fan_in)).
* ``small``         T=2048, d=512, d_ff=1376, E=4, K=2, 1 shared, bf16, top-K
                    then softmax over the K; b ~ N(0, 0.01); weights N(0, 0.02).
* ``medium``        T=8192, d=2048, d_ff=1408, E=64, K=8, 2 shared, bf16;
                    router rows scaled by load rank to give a Zipf-like skew
                    with 4 experts forced empty.
* ``large_prefill`` T=16384, d=7168, d_ff=2048, E=256, K=8, 2 shared, bf16;
                    weights and router N(0, 0.006); zero bias.
* ``large_decode``  the same layer at T=64.
* ``latent``        8192 tokens (B=2 x 4096), M=4096, latent L=1024, I=512,
                    E=128, K=8, sigmoid scores + bias N(0, 0.05) select the
                    top-(K+1); weights are the raw sigmoid scores (no
                    renormalisation); RMSNorm in L (eps 1e-6, gamma 1); one
                    shared FFN of width 2048 at width M; weights N(0, 0.02).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "generate", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "expert_seed", "ZIPF_ALPHA", "ZIPF_EMPTY",
]

# Slots of the root SeedSequence; the order is part of the input definition.
_SLOT_X, _SLOT_X_DECODE, _SLOT_ROUTER, _SLOT_BIAS, _SLOT_EXPERTS, _SLOT_SHARED, \
    _SLOT_LAT_DOWN, _SLOT_LAT_UP, _SLOT_ZIPF = range(9)
_N_SLOTS = 9

# Router-row scale exponent and forced-empty count of the skewed workload.
# Scaling the N(0, 0.02) router row of the expert with load rank r by
# r**-0.8 gives realised loads whose log-log slope against rank is about
# -1.1 for 8192 tokens, top-8 of 64 (calibrated offline by simulation, and
# re-measured through the oracle by the test suite). A zero row (logit = bias
# only, |b| ~ 0.01) loses to at least 8 of the 60 experts whose logits have
# std >= 0.02 * sqrt(2048) * 60**-0.8 for every realistic draw, so those 4
# experts receive no tokens.
ZIPF_ALPHA = 0.8
ZIPF_EMPTY = 4


@dataclass(frozen=True)
class Workload:
    name: str
    config_no: int
    T: int
    d: int            # model width (M for the latent workload)
    d_ff: int         # per-expert intermediate width (I for latent)
    E: int
    K: int
    n_shared: int
    d_ff_shared: int  # width of ONE shared FFN
    latent: int       # 0, or L (routed experts run at width L)
    act: str          # "f32" or "bf16": x, expert/shared/latent weights, out
    route: str        # "topk_softmax" | "softmax_topk" | "sigmoid_bias"
    renormalize: bool = False
    has_rmsnorm: bool = False
    rms_eps: float = 1e-6
    routed_scale: float = 1.0
    x_std: float = 1.0
    w_dist: str = "normal"      # "normal" or "uniform_fan_in"
    w_std: float = 0.02
    router_std: float = 0.02
    bias_std: float = 0.0       # 0 -> no bias (all zeros)
    router_skew: bool = False   # Zipf-like skew of router rows
    x_slot: int = _SLOT_X

    @property
    def d_e(self) -> int:
        """Width the routed experts run at."""
        return self.latent if self.latent else self.d

    @property
    def d_shared(self) -> int:
        return self.n_shared * self.d_ff_shared

    @property
    def rows(self) -> int:
        return self.T * self.K

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 1, T=128, d=64, d_ff=128, E=8, K=2, n_shared=1,
                 d_ff_shared=128, latent=0, act="f32", route="softmax_topk",
                 w_dist="uniform_fan_in"),
        Workload("small", 2, T=2048, d=512, d_ff=1376, E=4, K=2, n_shared=1,
                 d_ff_shared=1376, latent=0, act="bf16", route="topk_softmax",
                 w_std=0.02, router_std=0.02, bias_std=0.01),
        Workload("medium", 3, T=8192, d=2048, d_ff=1408, E=64, K=8, n_shared=2,
                 d_ff_shared=1408, latent=0, act="bf16", route="topk_softmax",
                 w_std=0.02, router_std=0.02, bias_std=0.01, router_skew=True),
        Workload("large_prefill", 4, T=16384, d=7168, d_ff=2048, E=256, K=8,
                 n_shared=2, d_ff_shared=2048, latent=0, act="bf16",
                 route="topk_softmax", w_std=0.006, router_std=0.006),
        Workload("large_decode", 4, T=64, d=7168, d_ff=2048, E=256, K=8,
                 n_shared=2, d_ff_shared=2048, latent=0, act="bf16",
                 route="topk_softmax", w_std=0.006, router_std=0.006,
                 x_slot=_SLOT_X_DECODE),
        Workload("latent", 5, T=8192, d=4096, d_ff=512, E=128, K=8, n_shared=1,
                 d_ff_shared=2048, latent=1024, act="bf16",
                 route="sigmoid_bias", renormalize=False, has_rmsnorm=True,
                 rms_eps=1e-6, w_std=0.02, router_std=0.02, bias_std=0.05),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even, returned as uint16 bits.

    Inputs are finite (every draw here is), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- seeding

def _root(w: Workload) -> list:
    return np.random.SeedSequence(1000 + w.config_no).spawn(_N_SLOTS)


def expert_seed(w: Workload, e: int, which: int) -> np.random.SeedSequence:
    """Seed of expert ``e``'s matrix ``which`` (0 gate, 1 up, 2 down)."""
    return _root(w)[_SLOT_EXPERTS].spawn(w.E)[e].spawn(3)[which]


def _rng(seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(seed, shape, w: Workload, kind: str, fan_in: int, std: float,
          out_bits: np.ndarray | None = None):
    """One weight/activation tensor: fp32 samples, then bf16 if act is bf16.

    kind: "act" (N(0, std)), "w" (the workload's weight law), "f32" (always
    fp32, N(0, std)).
    """
    g = _rng(seed)
    n = int(np.prod(shape))
    if kind == "w" and w.w_dist == "uniform_fan_in":
        bound = 1.0 / math.sqrt(fan_in)
        v = g.uniform(-bound, bound, size=n).astype(np.float32)
    else:
        v = g.standard_normal(size=n, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
    v = v.reshape(shape)
    if kind == "f32" or w.act == "f32":
        return v
    bits = f32_to_bf16_bits(v)
    if out_bits is not None:
        out_bits[...] = bits
        return out_bits
    return bits


def router_rows_scale(w: Workload) -> np.ndarray:
    """Per-expert multiplier of the router rows (all ones unless skewed)."""
    s = np.ones(w.E, dtype=np.float64)
    if not w.router_skew:
        return s
    perm = _rng(_root(w)[_SLOT_ZIPF]).permutation(w.E)
    s[perm[:ZIPF_EMPTY]] = 0.0
    ranks = np.arange(1, w.E - ZIPF_EMPTY + 1, dtype=np.float64)
    s[perm[ZIPF_EMPTY:]] = ranks ** (-ZIPF_ALPHA)
    return s


def generate(w: Workload, *, experts: bool = True, threads: int | None = None) -> dict:
    """Draw every input of workload ``w`` as host numpy arrays.

    Returns a dict with: x [T,d]; w_router [E,d] f32; bias [E] f32 or None;
    w_gate, w_up [E,d_ff,d_e]; w_down [E,d_e,d_ff]; ws_gate, ws_up
    [d_shared,d]; ws_down [d,d_shared] (the n_shared FFNs concatenated along
    the intermediate axis); and for the latent workload w_lat_down [L,d],
    w_lat_up [d,L], rms_gamma [L] f32. bf16 tensors are uint16 bit arrays.
    ``experts=False`` skips the routed expert weights (for routing-only use).
    """
    root = _root(w)
    nt = threads or _n_threads()
    out: dict = {"workload": w}
    out["x"] = _draw(root[w.x_slot], (w.T, w.d), w, "act", w.d, w.x_std)
    rscale = router_rows_scale(w)
    if w.w_dist == "uniform_fan_in":
        wr = _rng(root[_SLOT_ROUTER]).uniform(
            -1 / math.sqrt(w.d), 1 / math.sqrt(w.d), size=(w.E, w.d)).astype(np.float32)
    else:
        wr = _rng(root[_SLOT_ROUTER]).standard_normal((w.E, w.d), dtype=np.float32)
        wr *= np.float32(w.router_std)
    wr *= rscale.astype(np.float32)[:, None]
    out["w_router"] = wr
    if w.bias_std > 0:
        out["bias"] = (_rng(root[_SLOT_BIAS]).standard_normal(w.E, dtype=np.float32)
                       * np.float32(w.bias_std))
    else:
        out["bias"] = None

    de, f = w.d_e, w.d_ff
    dt = np.float32 if w.act == "f32" else np.uint16
    if experts:
        gate = np.empty((w.E, f, de), dtype=dt)
        up = np.empty((w.E, f, de), dtype=dt)
        down = np.empty((w.E, de, f), dtype=dt)
        eroot = root[_SLOT_EXPERTS].spawn(w.E)

        def one(e):
            s = eroot[e].spawn(3)
            gate[e] = _draw(s[0], (f, de), w, "w", de, w.w_std)
            up[e] = _draw(s[1], (f, de), w, "w", de, w.w_std)
            down[e] = _draw(s[2], (de, f), w, "w", f, w.w_std)

        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(one, range(w.E)))
        out["w_gate"], out["w_up"], out["w_down"] = gate, up, down

    if w.n_shared:
        fs = w.d_ff_shared
        sroot = root[_SLOT_SHARED].spawn(w.n_shared)
        parts = []
        for s_i in range(w.n_shared):
            s = sroot[s_i].spawn(3)
            parts.append((_draw(s[0], (fs, w.d), w, "w", w.d, w.w_std),
                          _draw(s[1], (fs, w.d), w, "w", w.d, w.w_std),
                          _draw(s[2], (w.d, fs), w, "w", fs, w.w_std)))
        out["ws_gate"] = np.ascontiguousarray(np.concatenate([p[0] for p in parts], 0))
        out["ws_up"] = np.ascontiguousarray(np.concatenate([p[1] for p in parts], 0))
        out["ws_down"] = np.ascontiguousarray(np.concatenate([p[2] for p in parts], 1))
    else:
        out["ws_gate"] = out["ws_up"] = out["ws_down"] = None

    if w.latent:
        L = w.latent
        out["w_lat_down"] = _draw(root[_SLOT_LAT_DOWN], (L, w.d), w, "w", w.d, w.w_std)
        out["w_lat_up"] = _draw(root[_SLOT_LAT_UP], (w.d, L), w, "w", L, w.w_std)
        out["rms_gamma"] = np.ones(L, dtype=np.float32)
    else:
        out["w_lat_down"] = out["w_lat_up"] = out["rms_gamma"] = None
    return out


def as_f64(a: np.ndarray, act: str) -> np.ndarray:
    """Exact fp64 values of a stored tensor (bf16 bits widened)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def draw_rows(seed: int, shape, act: str, std: float = 1.0) -> np.ndarray:
    """Extra seeded N(0, std) tensor (e.g. stand-in expert outputs for checking
    a later stage alone), fp32 or bf16 bits."""
    v = _rng(np.random.SeedSequence(seed)).standard_normal(int(np.prod(shape)), dtype=np.float32)
    v = (v * np.float32(std)).reshape(shape)
    return v if act == "f32" else f32_to_bf16_bits(v)
