"""Small custom layers for the tests, drawn through moe_synth's seeded generator."""
from __future__ import annotations

import numpy as np

import moe_synth
from moe_synth import Workload


def custom(name="custom", config_no=900, **kw) -> Workload:
    base = dict(T=37, d=24, d_ff=40, E=6, K=2, n_shared=2, d_ff_shared=16, latent=0,
                act="f32", route="topk_softmax", w_std=0.3, router_std=0.3, bias_std=0.05)
    base.update(kw)
    return Workload(name, config_no, **base)


def f64(a):
    """Exact fp64 value of a stored tensor (fp32, or bf16 bits)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return moe_synth.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def max_abs_rel(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)
