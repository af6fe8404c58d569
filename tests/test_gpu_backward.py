"""GPU parity of moe_backward against the CPU oracle's backward: input
gradient, router, expert and shared weight gradients, on the same seeded
inputs and output gradient; inactive experts' gradients left untouched."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import mixture_experts_ffn_fp32_amd as moe
import moe_synth
import oracle
from _gpu import f64, gpu_route, layer_of, need_gpu, sample_tokens, say, torch
from _layers import custom, max_abs_rel

pytestmark = pytest.mark.gpu

TOL = 2e-2  # max-abs-rel per gradient tensor: bf16 operands, fp32 accumulation
TOL_BY_ACT = {"bf16": TOL, "f32": 1e-5}  # fp32: every product in fp32

SHAPES = {"w_router": ("E", "d"), "w_gate": ("E", "d_ff", "de"), "w_up": ("E", "d_ff", "de"),
          "w_down": ("E", "de", "d_ff"), "ws_gate": ("d_shared", "d"),
          "ws_up": ("d_shared", "d"), "ws_down": ("d", "d_shared"),
          "w_lat_down": ("L", "d"), "w_lat_up": ("d", "L"), "rms_gamma": ("L",)}


def _keys(w):
    return [k for k in SHAPES if (w.d_shared or not k.startswith("ws_"))
            and (w.latent or k not in ("w_lat_down", "w_lat_up", "rms_gamma"))
            and (w.has_rmsnorm or k != "rms_gamma")]


def _grad_buffers(w, keys):
    dims = {"E": w.E, "d": w.d, "d_ff": w.d_ff, "d_shared": w.d_shared, "L": w.latent,
            "de": w.latent or w.d}
    return {k: torch.full(tuple(dims[s] for s in SHAPES[k]), float("nan"), dtype=torch.float32,
                          device="cuda") for k in keys}


def _d_out(w, seed):
    v = moe_synth.draw_rows(seed, (w.T, w.d), w.act)
    t = torch.from_numpy(v)
    return v, (t.view(torch.bfloat16) if w.act == "bf16" else t).cuda()


def run_backward(w, a, layer, keys, seed=11):
    bits, dy = _d_out(w, seed)
    grads = _grad_buffers(w, keys)
    dx = layer.backward(layer.dev["x"], dy, grads=grads)
    torch.cuda.synchronize()
    g_idx = gpu_route(layer)[0]
    return bits, f64(dx), {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}, g_idx


def oracle_selection(orc, g_idx):
    """The oracle's selection, with the GPU's on near-tied tokens (both are
    correct there)."""
    o_idx, _, gap, _ = orc.route()
    use = o_idx.copy()
    near = gap < moe.TIE_EPS
    use[near] = g_idx[near]
    return use, int(near.sum())


def oracle_backward_chunked(orc, dy, use, tokens, n_chunks, **kw):
    """The oracle's backward over `tokens` as n_chunks calls run side by side
    (its weight-gradient path is serial within a call): dx rows in token
    order, weight gradients the chunks' sums added in chunk order (every
    gradient is a sum of per-token terms)."""
    parts = [p for p in np.array_split(np.asarray(tokens), n_chunks) if len(p)]

    def one(part):
        return orc.backward(dy[part], tokens=part, idx_override=use[part], **kw)

    ref = None
    with ThreadPoolExecutor(min(16, len(parts))) as ex:
        for r in ex.map(one, parts):
            if ref is None:
                ref = r
                continue
            ref["dx"] = np.concatenate([ref["dx"], r["dx"]])
            for k in r:
                if k != "dx":
                    ref[k] += r[k]
    return ref


def check_all(w, a, layer, keys=None, seed=11, tol=None):
    keys = _keys(w) if keys is None else keys
    tol = tol or TOL_BY_ACT[w.act]
    bits, dx, grads, g_idx = run_backward(w, a, layer, keys, seed)
    orc = oracle.Oracle(w, a)
    use, n_near = oracle_selection(orc, g_idx)
    ref = oracle_backward_chunked(orc, moe_synth.as_f64(bits, w.act), use, np.arange(w.T),
                                  max(1, min(16, w.T // 32)), shared=bool(w.d_shared))
    errs = {"dx": max_abs_rel(dx, ref["dx"])}
    active = np.bincount(use.ravel(), minlength=w.E) > 0
    for k in keys:
        got = grads[k]
        if k in ("w_gate", "w_up", "w_down"):
            assert np.all(np.isnan(got[~active])), f"{k}: inactive experts were written"
            assert np.all(np.isfinite(got[active])), k
            errs[k] = max_abs_rel(got[active], ref[k][active])
        else:
            assert np.all(np.isfinite(got)), k
            errs[k] = max_abs_rel(got, ref[k])
    say(f"  backward {w.name}: T={w.T} near-ties={n_near} active={int(active.sum())}/{w.E} "
        + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, (k, v)
    return errs


LAYERS = {
    "small_256": None,
    "tiny": None,  # the fp32 workload (generic kernel, fp32 matrix cores)
    "latent_f32": dict(T=64, d=64, latent=32, d_ff=32, E=4, K=2, act="f32",
                       route="sigmoid_bias", bias_std=0.1, has_rmsnorm=True, n_shared=1,
                       d_ff_shared=32, w_std=0.1, router_std=0.1),
    "f32_ragged": dict(T=300, d=96, d_ff=160, E=6, K=2, act="f32", n_shared=1,
                       d_ff_shared=64, w_std=0.08, router_std=0.08),
    # few rows per expert: the products read W_down, W_gate, W_up (and the
    # shared / latent projections) in place, K-major
    "decode_like": dict(T=64, d=256, d_ff=384, E=32, K=4, act="bf16", n_shared=1,
                        d_ff_shared=128, w_std=0.05, router_std=0.05, bias_std=0.01),
    "decode_dff_mod32": dict(T=48, d=128, d_ff=160, E=16, K=2, act="bf16", n_shared=1,
                             d_ff_shared=96, w_std=0.08, router_std=0.08),
    "decode_latent": dict(T=32, d=128, latent=64, d_ff=64, E=8, K=2, act="bf16",
                          route="sigmoid_bias", bias_std=0.05, has_rmsnorm=True, n_shared=1,
                          d_ff_shared=64, w_std=0.08, router_std=0.08),
    "topk_e16": dict(T=512, d=256, d_ff=384, E=16, K=4, act="bf16", n_shared=1,
                     d_ff_shared=256, w_std=0.05, router_std=0.05, bias_std=0.01),
    "softmax_first": dict(T=300, d=128, d_ff=160, E=8, K=2, act="bf16", route="softmax_topk",
                          n_shared=1, d_ff_shared=96, w_std=0.08, router_std=0.08),
    "sigmoid_renorm": dict(T=300, d=128, d_ff=96, E=12, K=3, act="bf16", route="sigmoid_bias",
                           renormalize=True, routed_scale=2.5, bias_std=0.1, n_shared=0,
                           d_ff_shared=0, w_std=0.08, router_std=0.08),
    "sigmoid_raw": dict(T=200, d=96, d_ff=64, E=6, K=2, act="bf16", route="sigmoid_bias",
                        bias_std=0.1, n_shared=2, d_ff_shared=32, w_std=0.1, router_std=0.1),
    "one_expert": dict(T=100, d=64, d_ff=96, E=1, K=1, act="bf16", n_shared=1, d_ff_shared=64,
                       w_std=0.1, router_std=0.1),
    "inactive": dict(T=6, d=64, d_ff=64, E=32, K=1, act="bf16", n_shared=0, d_ff_shared=0,
                     w_std=0.1, router_std=0.1),
    "k_eq_e": dict(T=150, d=64, d_ff=64, E=4, K=4, act="bf16", w_std=0.1, router_std=0.1,
                   n_shared=1, d_ff_shared=32),
    # StableLatentMoE layers: routed experts in width L between the projections
    "latent_norm_sigmoid": dict(T=300, d=128, latent=64, d_ff=96, E=8, K=3, act="bf16",
                                route="sigmoid_bias", bias_std=0.05, has_rmsnorm=True,
                                n_shared=1, d_ff_shared=160, w_std=0.08, router_std=0.08),
    "latent_nonorm_topk": dict(T=200, d=96, latent=64, d_ff=64, E=6, K=2, act="bf16",
                               has_rmsnorm=False, n_shared=0, d_ff_shared=0, w_std=0.1,
                               router_std=0.1),
    # large experts (d x d_ff = 2^23) with ~256 rows each: the products read
    # W_down, W_gate and W_up in place on the 2x4-wavefront tile, with
    # partial m-tiles; every gradient compared in full
    "kmajor_large_expert": dict(T=512, d=4096, d_ff=2048, E=4, K=2, act="bf16", n_shared=1,
                                d_ff_shared=512, w_std=0.02, router_std=0.02, bias_std=0.01),
}

# layers whose backward must take the in-place (K-major) weight products
IN_PLACE = {"kmajor_large_expert": 3, "decode_like": 3}
# seeds: layers added later take their own, so the others keep theirs
SEED_OF = {"kmajor_large_expert": 980}
_SEEDED = sorted(n for n in LAYERS if n not in SEED_OF)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("name", sorted(LAYERS))
def test_backward_matches_oracle(name):
    if name == "small_256":
        w = moe_synth.get("small").with_T(256)
    elif name == "tiny":
        w = moe_synth.get("tiny")
    else:
        cfg = SEED_OF.get(name) or 950 + _SEEDED.index(name)
        w = custom(name, config_no=cfg, **LAYERS[name])
    say(f"case backward {name} T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} K={w.K} route={w.route}")
    if name in IN_PLACE:
        assert moe.moe_plan(moe.make_desc(w))["backward_in_place"] == IN_PLACE[name]
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    check_all(w, a, layer)


def test_backward_is_deterministic_and_partial_requests():
    """Two calls give the same bits; gradients not asked for are not
    written, the ones asked for are unchanged."""
    w = custom("bwd_det", config_no=990, **LAYERS["topk_e16"])
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    _, dy = _d_out(w, 3)
    g1 = _grad_buffers(w, _keys(w))
    g2 = _grad_buffers(w, ["w_down", "ws_up"])
    dx1 = layer.backward(layer.dev["x"], dy, grads=g1).clone()
    dx2 = layer.backward(layer.dev["x"], dy, grads=g2)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2)
    assert torch.equal(g1["w_down"].nan_to_num(7.0), g2["w_down"].nan_to_num(7.0))
    assert torch.equal(g1["ws_up"], g2["ws_up"])


@pytest.mark.timeout(900)
def test_backward_persistent_edges():
    """The recomputed gate/up pre-activations on the persistent kernel's fp32
    gate/up epilogue at its edges: reduction ending 32 columns into a stage
    (d = 2080), a partial last n-tile (d_ff = 1056 = 8 x 128 + 32), skewed
    experts (0, 1 and all tokens) and a partial last dense m-tile in the
    shared recompute (T = 8229): input gradients on a token sample, and the
    weight gradients of the smallest non-empty expert (one row)."""
    w = custom(name="persist_bwd", config_no=640, T=8229, d=2080, d_ff=1056, E=8, K=4,
               act="bf16", n_shared=1, d_ff_shared=2048, route="sigmoid_bias", bias_std=1.0,
               w_std=0.03, router_std=0.03)
    say("case backward persistent edges: generating inputs")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    bits, dx, grads, g_idx = run_backward(w, a, layer, ["w_gate", "w_up", "w_down"])
    orc = oracle.Oracle(w, a)
    use, n_near = oracle_selection(orc, g_idx)
    dy = moe_synth.as_f64(bits, w.act)
    # the last 37 tokens fill the shared recompute's partial last m-tile; each
    # expert's last 16 tokens sit in its own last m-tile
    tails = [np.nonzero((use == e).any(1))[0][-16:] for e in range(w.E)]
    toks = np.union1d(sample_tokens(use, w.E, 256, seed=7),
                      np.concatenate([np.arange(w.T - 37, w.T)] + tails))
    ref = orc.backward(dy[toks], tokens=toks, idx_override=use[toks], experts=None,
                       router=False, shared=False)
    err = max_abs_rel(dx[toks], ref["dx"])
    counts = np.bincount(use.ravel(), minlength=w.E)
    nz = np.nonzero(counts)[0]
    e = int(nz[np.argmin(counts[nz])])
    mine = np.nonzero((use == e).any(1))[0]
    one = orc.backward(dy[mine], tokens=mine, idx_override=use[mine], experts=e, router=False,
                       shared=False)
    errs = {k: max_abs_rel(grads[k][e], one[k][0]) for k in ("w_gate", "w_up", "w_down")}
    assert np.all(np.isnan(grads["w_gate"][counts == 0]))
    say(f"  persistent edges: loads {counts.tolist()} near-ties={n_near} "
        f"dx(sample {len(toks)})={err:.2e} expert {e} ({counts[e]} rows): "
        + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert err <= TOL
    for v in errs.values():
        assert v <= TOL
    del layer, a
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_backward_medium_sampled():
    """Full-size medium layer (skewed loads, empty experts): input gradients on
    a seeded token sample, and the weight gradients of the smallest non-empty
    expert over all of its tokens."""
    w = moe_synth.get("medium")
    say("case backward medium: generating inputs")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    bits, dx, grads, g_idx = run_backward(w, a, layer, ["w_gate", "w_up", "w_down"])
    orc = oracle.Oracle(w, a)
    use, n_near = oracle_selection(orc, g_idx)
    dy = moe_synth.as_f64(bits, w.act)
    toks = sample_tokens(use, w.E, 256, seed=5)
    ref = orc.backward(dy[toks], tokens=toks, idx_override=use[toks], experts=None,
                       router=False, shared=False)
    err = max_abs_rel(dx[toks], ref["dx"])
    counts = np.bincount(use.ravel(), minlength=w.E)
    nz = np.nonzero(counts)[0]
    e = int(nz[np.argmin(counts[nz])])
    mine = np.nonzero((use == e).any(1))[0]
    one = orc.backward(dy[mine], tokens=mine, idx_override=use[mine], experts=e, router=False,
                       shared=False)
    errs = {k: max_abs_rel(grads[k][e], one[k][0]) for k in ("w_gate", "w_up", "w_down")}
    assert np.all(np.isnan(grads["w_gate"][counts == 0]))
    say(f"  medium: near-ties={n_near} dx(sample {len(toks)})={err:.2e} expert {e} "
        f"({counts[e]} rows): " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert err <= TOL
    for v in errs.values():
        assert v <= TOL
    del layer, a
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["large_decode", "large_prefill"])
def test_backward_large_full_size_sampled(name):
    """Full-size large layers (decode: 64 tokens over 256 experts; prefill:
    16384 tokens; both read the expert weights in place, K-major): input
    gradients on a seeded sample of 256 tokens, and (decode) the weight
    gradients of the smallest non-empty expert over its tokens. (The prefill
    layer's weight gradients: the masked test below.)"""
    w = moe_synth.get(name)
    say(f"case backward {name}: generating inputs")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    say(f"  {name}: backward")
    bits, d_out = _d_out(w, 11)
    dev = _grad_buffers(w, ["w_gate", "w_up", "w_down"])  # up to 45 GB: copied back per expert
    dx = f64(layer.backward(layer.dev["x"], d_out, grads=dev))
    torch.cuda.synchronize()
    g_idx = gpu_route(layer)[0]
    orc = oracle.Oracle(w, a)
    say(f"  {name}: oracle routing")
    use, n_near = oracle_selection(orc, g_idx)
    dy = moe_synth.as_f64(bits, w.act)
    toks = np.sort(np.random.default_rng(7).choice(w.T, size=min(w.T, 256), replace=False))
    say(f"  {name}: oracle input gradients of {len(toks)} tokens")
    ref = orc.backward(dy[toks], tokens=toks, idx_override=use[toks], experts=None,
                       router=False, shared=False)
    err = max_abs_rel(dx[toks], ref["dx"])
    counts = np.bincount(use.ravel(), minlength=w.E)
    nz = np.nonzero(counts)[0]
    e = int(nz[np.argmin(counts[nz])])
    mine = np.nonzero((use == e).any(1))[0]
    errs = {}
    if len(mine) <= 64:
        say(f"  {name}: oracle weight gradients of expert {e} over its {len(mine)} tokens")
        one = orc.backward(dy[mine], tokens=mine, idx_override=use[mine], experts=e,
                           router=False, shared=False)
        errs = {k: max_abs_rel(dev[k][e].cpu().numpy().astype(np.float64), one[k][0])
                for k in ("w_gate", "w_up", "w_down")}
    say(f"  {name}: near-ties={n_near} dx(sample {len(toks)})={err:.2e} expert {e} "
        f"({counts[e]} rows): " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert err <= TOL
    for v in errs.values():
        assert v <= TOL
    del layer, a, dev
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_backward_latent_full_size_sampled():
    """Full-size latent layer (sigmoid routing, RMSNorm in L): input gradients
    on a seeded token sample and the weight gradients of the smallest
    non-empty expert over its tokens. (The projections' and the gain's
    gradients: the masked test below.)"""
    w = moe_synth.get("latent")
    say("case backward latent: generating inputs")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    bits, dx, grads, g_idx = run_backward(w, a, layer, ["w_gate", "w_up", "w_down"])
    orc = oracle.Oracle(w, a)
    use, n_near = oracle_selection(orc, g_idx)
    dy = moe_synth.as_f64(bits, w.act)
    toks = sample_tokens(use, w.E, 128, seed=6)
    ref = orc.backward(dy[toks], tokens=toks, idx_override=use[toks], experts=None,
                       router=False, shared=False, latent=False)
    err = max_abs_rel(dx[toks], ref["dx"])
    counts = np.bincount(use.ravel(), minlength=w.E)
    nz = np.nonzero(counts)[0]
    e = int(nz[np.argmin(counts[nz])])
    mine = np.nonzero((use == e).any(1))[0]
    one = orc.backward(dy[mine], tokens=mine, idx_override=use[mine], experts=e, router=False,
                       shared=False, latent=False)
    errs = {k: max_abs_rel(grads[k][e], one[k][0]) for k in ("w_gate", "w_up", "w_down")}
    say(f"  latent: near-ties={n_near} dx(sample {len(toks)})={err:.2e} expert {e} "
        f"({counts[e]} rows): " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert err <= TOL
    for v in errs.values():
        assert v <= TOL
    del layer, a
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_backward_large_decode_router_shared_and_expert():
    """Full-size decode layer (64 tokens over 256 experts; every weight read
    in place): router and shared weight gradients over all tokens, and the
    most loaded expert's weight gradients, element by element."""
    w = moe_synth.get("large_decode")
    say("case backward large_decode (router, shared, expert): generating inputs")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    keys = ["w_router", "ws_gate", "ws_up", "ws_down", "w_gate", "w_up", "w_down"]
    bits, d_out = _d_out(w, 19)
    dev = _grad_buffers(w, keys)  # expert buffers up to 45 GB: copied back for one expert
    dx = f64(layer.backward(layer.dev["x"], d_out, grads=dev))
    torch.cuda.synchronize()
    g_idx = gpu_route(layer)[0]
    orc = oracle.Oracle(w, a)
    use, n_near = oracle_selection(orc, g_idx)
    counts = np.bincount(use.ravel(), minlength=w.E)
    e = int(np.argmax(counts))
    got = {k: (dev[k][e] if k in ("w_gate", "w_up", "w_down") else dev[k]).cpu().numpy()
           .astype(np.float64) for k in keys}
    del dev
    torch.cuda.empty_cache()
    dy = moe_synth.as_f64(bits, w.act)
    say(f"  large_decode: oracle backward over {w.T} tokens (expert {e}: {counts[e]} rows)")
    ref = oracle_backward_chunked(orc, dy, use, np.arange(w.T), 16, experts=e, router=True,
                                  shared=True)
    errs = {"dx": max_abs_rel(dx, ref["dx"])}
    for k in keys:
        errs[k] = max_abs_rel(got[k], ref[k][0] if k in ("w_gate", "w_up", "w_down") else ref[k])
    say(f"  large_decode: near-ties={n_near} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    del layer, a
    torch.cuda.empty_cache()


def _masked_backward(name, in_place=None):
    """The full-size layer `name` with an output gradient that is zero
    outside a token set S: S = every token of one expert holding 257-511
    rows (a full and a partial 256-row m-tile) plus a seeded sample of 32
    others. Each token's gradient terms are independent of the other tokens,
    so every weight gradient is then the oracle's sum over S: router, shared
    (and latent projections and RMSNorm gain) gradients and that expert's
    gate/up/down are compared element by element; dx matches on S and is
    exactly zero elsewhere."""
    w = moe_synth.get(name)
    say(f"case backward {name} masked: generating inputs")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    if in_place is not None:
        assert moe.moe_plan(layer.desc)["backward_in_place"] == in_place
    g_idx = gpu_route(layer)[0]
    orc = oracle.Oracle(w, a)
    say(f"  {name} masked: oracle routing")
    use, n_near = oracle_selection(orc, g_idx)
    counts = np.bincount(use.ravel(), minlength=w.E)
    mid = np.nonzero((counts > 256) & (counts < 512))[0]
    assert len(mid), "no expert with a partial second m-tile"
    e = int(mid[np.argmin(counts[mid])])
    mine = np.nonzero((use == e).any(1))[0]
    rng = np.random.default_rng(13)
    others = rng.choice(np.setdiff1d(np.arange(w.T), mine), size=32, replace=False)
    S = np.sort(np.union1d(mine, others))
    bits = moe_synth.draw_rows(17, (w.T, w.d), w.act)
    mask = np.zeros(w.T, bool)
    mask[S] = True
    bits[~mask] = 0  # +0.0 in bf16
    dy_dev = torch.from_numpy(bits).view(torch.bfloat16).cuda()
    keys = _keys(w)
    grads = _grad_buffers(w, keys)
    say(f"  {name} masked: backward (expert {e}: {counts[e]} rows, |S| = {len(S)})")
    dx = f64(layer.backward(layer.dev["x"], dy_dev, grads=grads))
    torch.cuda.synchronize()
    got = {k: (grads[k][e].cpu().numpy() if k in ("w_gate", "w_up", "w_down")
               else grads[k].cpu().numpy()).astype(np.float64) for k in keys}
    del grads
    torch.cuda.empty_cache()
    dy = moe_synth.as_f64(bits, w.act)
    say(f"  {name} masked: oracle backward over {len(S)} tokens in 32 chunks")
    ref = oracle_backward_chunked(orc, dy, use, S, 32, experts=e, router=True, shared=True)
    errs = {"dx": max_abs_rel(dx[S], ref["dx"])}
    for k in keys:
        errs[k] = max_abs_rel(got[k], ref[k][0] if k in ("w_gate", "w_up", "w_down") else ref[k])
    say(f"  {name} masked: near-ties={n_near} "
        + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert np.all(dx[~mask] == 0)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    del layer, a
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_backward_large_prefill_masked_output_gradient():
    """Full-size large prefill layer (16384 tokens, the launch configuration
    the benchmark times; expert weights read in place) under a masked output
    gradient: router, shared and one expert's weight gradients element by
    element."""
    _masked_backward("large_prefill", in_place=3)


@pytest.mark.timeout(900)
def test_backward_medium_masked_output_gradient():
    """Full-size medium layer (skewed loads, empty experts, two shared
    experts) under a masked output gradient: router, shared and one expert's
    weight gradients element by element."""
    _masked_backward("medium")


@pytest.mark.timeout(900)
def test_backward_latent_masked_output_gradient():
    """Full-size latent layer (sigmoid routing, RMSNorm in L) under a masked
    output gradient: the latent down- and up-projection, RMSNorm gain,
    router, shared and one expert's weight gradients element by element."""
    _masked_backward("latent")
