"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import mixture_experts_ffn_fp32_amd as moe
import oracle
from _layers import max_abs_rel

torch = pytest.importorskip("torch")

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max-abs-rel of layer outputs
G_TOL = 1e-5                        # routing weights (fp32 router)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def dev_of(arrays):
    return moe.to_device(arrays, "cuda")


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def layer_of(w, arrays, dev=None):
    return moe.Layer(w, dev if dev is not None else dev_of(arrays), device="cuda")


def gpu_route(layer):
    w = layer.spec
    dv = "cuda"
    idx = torch.full((w.T, w.K), -7, dtype=torch.int32, device=dv)
    g = torch.full((w.T, w.K), -7.0, dtype=torch.float32, device=dv)
    gap = torch.full((w.T,), -7.0, dtype=torch.float32, device=dv)
    top = torch.full((w.T, w.K + 1), -7.0, dtype=torch.float32, device=dv)
    moe.moe_route(layer.desc, layer.weights, layer.dev["x"], idx, g, gap, top, layer.ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), g.cpu().numpy(), gap.cpu().numpy(), top.cpu().numpy()


def check_route(w, arrays, layer, orc=None):
    """idx bit-exact where the oracle's gap >= 1e-5; weights, gaps and top
    scores within 1e-5 where the selections agree. Returns the oracle route."""
    orc = orc or oracle.Oracle(w, arrays)
    o_idx, o_g, o_gap, o_top = orc.route()
    g_idx, g_g, g_gap, g_top = gpu_route(layer)
    far = o_gap >= moe.TIE_EPS
    assert np.array_equal(g_idx[far], o_idx[far]), f"{(g_idx[far] != o_idx[far]).any(1).sum()} tokens differ"
    same = np.all(g_idx == o_idx, axis=1)
    assert same[far].all()
    assert np.max(np.abs(g_g[same] - o_g[same]), initial=0) <= G_TOL
    fin = same & np.isfinite(o_gap)
    assert np.max(np.abs(g_gap[fin] - o_gap[fin]), initial=0) <= G_TOL
    assert np.all(np.isinf(g_gap[~np.isfinite(o_gap)]))
    tf = np.isfinite(o_top) & same[:, None]
    assert np.max(np.abs(g_top[tf] - o_top[tf]), initial=0) <= G_TOL
    say(f"  route {w.name}: T={w.T} near-ties(oracle)={int((~far).sum())}")
    return o_idx, o_g, o_gap, g_idx


def check_forward(w, arrays, layer, tokens=None, orc=None, o_route=None, tol=None):
    """Layer output within max-abs-rel tol of the oracle on `tokens` (all if
    None). Tokens the oracle finds near-tied are re-evaluated by the oracle
    with the GPU's own selection. Counts bit-exact against the dispatch of
    the selection actually used."""
    tol = tol or TOL[w.act]
    orc = orc or oracle.Oracle(w, arrays)
    counts = torch.full((w.E,), -1, dtype=torch.int32, device="cuda")
    ntie = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    out = layer.forward(layer.dev["x"], counts=counts, n_near_ties=ntie)
    torch.cuda.synchronize()
    got = f64(out)
    if o_route is None:
        o_idx, _, o_gap, g_idx = check_route(w, arrays, layer, orc)
    else:
        o_idx, _, o_gap, g_idx = o_route
    near = o_gap < moe.TIE_EPS
    use = o_idx.copy()
    use[near] = g_idx[near]
    cnt = np.bincount(use.ravel(), minlength=w.E)
    assert np.array_equal(counts.cpu().numpy(), cnt)
    assert int(ntie.item()) >= 0
    toks = np.arange(w.T) if tokens is None else np.asarray(tokens)
    ref, r_idx, _, _ = orc.forward(tokens=toks, idx_override=use[toks])
    err = max_abs_rel(got[toks], ref)
    say(f"  forward {w.name}: T={w.T} checked={len(toks)} max-abs-rel={err:.3e} tol={tol}")
    assert err <= tol, err
    assert np.all(np.isfinite(got))
    return got, ref, toks, use


def sample_tokens(idx, E, n, seed=0):
    """Seeded sample of n tokens that includes every token of the smallest
    non-empty expert and up to 64 tokens of the largest."""
    T = idx.shape[0]
    rng = np.random.default_rng(seed)
    counts = np.bincount(idx.ravel(), minlength=E)
    nz = np.nonzero(counts)[0]
    small = nz[np.argmin(counts[nz])]
    big = np.argmax(counts)
    must = np.nonzero((idx == small).any(1))[0]
    bigt = np.nonzero((idx == big).any(1))[0]
    must = np.union1d(must, rng.choice(bigt, size=min(64, len(bigt)), replace=False))
    rest = np.setdiff1d(np.arange(T), must)
    extra = rng.choice(rest, size=max(0, min(len(rest), n - len(must))), replace=False)
    return np.sort(np.union1d(must, extra))
