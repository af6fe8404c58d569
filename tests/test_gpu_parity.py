"""GPU parity of every C-ABI entry point against the CPU oracle, on small
and edge-case layers (full-size workloads are in test_gpu_full.py)."""
import numpy as np
import pytest

import mixture_experts_ffn_fp32_amd as moe
import moe_synth
import oracle
from _gpu import (TOL, check_forward, check_route, dev_of, f64, layer_of, need_gpu,
                  sample_tokens, say, torch)
from _layers import custom, max_abs_rel

pytestmark = pytest.mark.gpu

EDGE = {
    "ragged_f32": dict(T=37, d=24, d_ff=40, E=6, K=2, act="f32"),
    "ragged_bf16": dict(T=53, d=40, d_ff=72, E=5, K=3, act="bf16"),
    "k_eq_e": dict(T=33, E=4, K=4),
    "one_expert": dict(T=29, E=1, K=1, n_shared=0, d_ff_shared=0),
    "k16": dict(T=70, d=32, d_ff=16, E=32, K=16, act="bf16"),
    "e1024": dict(T=40, d=16, d_ff=8, E=1024, K=2, n_shared=1, d_ff_shared=8),
    "softmax_first": dict(T=100, E=9, K=3, route="softmax_topk"),
    "sigmoid": dict(T=90, E=12, K=4, route="sigmoid_bias", bias_std=0.2),
    "sigmoid_renorm_scaled": dict(T=90, E=12, K=4, route="sigmoid_bias", bias_std=0.2,
                                  renormalize=True, routed_scale=2.5, act="bf16"),
    "latent_f32": dict(T=45, d=32, latent=16, d_ff=24, E=7, K=3, route="sigmoid_bias",
                       has_rmsnorm=True, n_shared=1, d_ff_shared=40),
    "latent_bf16_noshared": dict(T=45, d=32, latent=24, d_ff=16, E=7, K=3, act="bf16",
                                 route="sigmoid_bias", has_rmsnorm=True, n_shared=0,
                                 d_ff_shared=0),
    "latent_nonorm": dict(T=30, d=24, latent=16, d_ff=8, E=5, K=2, has_rmsnorm=False),
    "no_shared_bf16": dict(T=300, d=64, d_ff=96, E=8, K=2, act="bf16", n_shared=0,
                           d_ff_shared=0),
    "many_chunks": dict(T=1537, d=32, d_ff=24, E=16, K=8, act="bf16"),
    "wide_bf16": dict(T=200, d=256, d_ff=520, E=8, K=2, act="bf16", w_std=0.05,
                      router_std=0.05),
    # few experts but a model too wide for the wavefront-per-token router
    "mfma_router": dict(T=1100, d=2560, d_ff=64, E=16, K=2, act="bf16", w_std=0.02,
                        router_std=0.02),
}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_workload_route_and_forward(name):
    w = moe_synth.get(name)
    say(f"case {name}")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    orc = oracle.Oracle(w, a)
    r = check_route(w, a, layer, orc)
    got, ref, toks, _ = check_forward(w, a, layer, orc=orc, o_route=r)
    if name == "tiny":
        # moe-from-scratch's allclose check of sorted dispatch vs the naive loop
        assert np.max(np.abs(got - ref)) <= 1e-5


# Pipelined-GEMM shapes: reductions ending 32 columns into a 64-column stage
# (d or d_ff = 32 mod 64), at sizes that pick each tile shape: few tiles
# (64x128 / 8-wavefront 128x128), 128x128 two per CU, 256x256.
TAIL = {
    "tail_few": (dict(T=300, d=96, d_ff=160, E=4, K=2, act="bf16", n_shared=1, d_ff_shared=160,
                      w_std=0.05, router_std=0.05), None),
    "tail_mid": (dict(T=4096, d=1056, d_ff=800, E=4, K=2, act="bf16", n_shared=1,
                      d_ff_shared=800, w_std=0.03, router_std=0.03), 512),
    "tail_big": (dict(T=8192, d=480, d_ff=1056, E=4, K=2, act="bf16", n_shared=1,
                      d_ff_shared=1056, w_std=0.03, router_std=0.03), 384),
}


@pytest.mark.parametrize("name", sorted(TAIL))
def test_pipelined_gemm_k_tail(name):
    kw, n = TAIL[name]
    w = custom(name=name, config_no=600 + sorted(TAIL).index(name), **kw)
    say(f"case k-tail {name} T={w.T} d={w.d} d_ff={w.d_ff}")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    orc = oracle.Oracle(w, a)
    r = check_route(w, a, layer, orc)
    toks = None if n is None else sample_tokens(r[0], w.E, n, seed=w.config_no)
    check_forward(w, a, layer, tokens=toks, orc=orc, o_route=r)
    plan = moe.moe_plan(layer.desc)
    say(f"  plan {plan}")
    assert plan["gate_up_pipelined"] and plan["down_pipelined"]
    # few tiles / merged 256x256 / separate 256x256
    want = {"tail_few": (1, 64), "tail_mid": (1, 256), "tail_big": (0, 256)}[name]
    assert (plan["merged_shared"], plan["gate_up_tile_m"]) == want


def test_persistent_grouped_gemms():
    """Both grouped GEMMs on the persistent kernel: reductions ending 32
    columns into a stage (2080 and 1056), a partial last n-tile in each
    (1056 = 8 x 128 + 32 SwiGLU columns, 2080 = 8 x 256 + 32), expert loads
    skewed by the router bias (partial m-tiles of many heights); the shared
    experts' dense gate/up (33 x 16 tiles) on it too, its last m-tile
    partial (8229 = 32 x 256 + 37 tokens)."""
    w = custom(name="persist", config_no=640, T=8229, d=2080, d_ff=1056, E=8, K=4, act="bf16",
               n_shared=1, d_ff_shared=2048, route="sigmoid_bias", bias_std=1.0, w_std=0.03,
               router_std=0.03)
    say(f"case persistent T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} K={w.K}")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    plan = moe.moe_plan(layer.desc)
    say(f"  plan {plan}")
    assert plan["persistent"] == 3
    orc = oracle.Oracle(w, a)
    r = check_route(w, a, layer, orc)
    counts = np.bincount(r[0].ravel(), minlength=w.E)
    say(f"  expert loads {counts.tolist()}")
    toks = sample_tokens(r[0], w.E, 384, seed=w.config_no)
    check_forward(w, a, layer, tokens=toks, orc=orc, o_route=r)


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_layer(name):
    w = custom(name=name, config_no=500 + sorted(EDGE).index(name), **EDGE[name])
    say(f"case edge {name}")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    check_forward(w, a, layer)


def test_all_tokens_to_one_expert():
    """BUG-08 of the APEX-1 docs: many tokens on one expert, others empty."""
    w = custom(name="hot", T=300, E=6, K=1, act="bf16", bias_std=0.0)
    a = moe_synth.generate(w)
    a["bias"] = np.zeros(w.E, np.float32)
    a["bias"][3] = 50.0
    say("case all tokens to expert 3")
    layer = layer_of(w, a)
    check_forward(w, a, layer)
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    layer.forward(layer.dev["x"], counts=counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0, 0, 300, 0, 0]


@pytest.mark.parametrize("E,K,lo,hi,kw", [
    (8, 3, 2, 5, {}),                                    # wavefront router, rank selection
    (64, 8, 3, 60, dict(act="bf16", d=2560, d_ff=64)),   # split-plane GEMM, rank selection
    (128, 8, 5, 69, {}),                                 # GEMM router, selection rounds; same lane
])
def test_exact_ties_take_lower_id(E, K, lo, hi, kw):
    """Experts lo and hi have identical router rows: equal logits, the lower id
    ranks first on both sides."""
    w = custom(name="ties", T=120, E=E, K=K, bias_std=0.0, **kw)
    a = moe_synth.generate(w)
    a["w_router"][hi] = a["w_router"][lo]
    a["bias"] = None
    layer = layer_of(w, a)
    say(f"case exact ties E={E} K={K} ids {lo}/{hi}")
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    g = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")
    moe.moe_route(layer.desc, layer.weights, layer.dev["x"], idx, g, ws=layer.ws)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    o_idx, _, _, _ = oracle.Oracle(w, a).route()
    both = (gi == lo).any(1) & (gi == hi).any(1)
    assert np.array_equal(gi, o_idx)
    one = ((gi == lo) | (gi == hi)).sum(1) == 1
    assert np.all((gi[one] == lo).any(1))
    assert both.sum() + one.sum() > 0


@pytest.mark.parametrize("T", [0, 1])
def test_tiny_token_counts(T):
    w = custom(name=f"t{T}", T=T, act="bf16")
    a = moe_synth.generate(w)
    say(f"case T={T}")
    layer = layer_of(w, a)
    counts = torch.full((w.E,), -1, dtype=torch.int32, device="cuda")
    ntie = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((max(T, 1), w.d), dtype=torch.bfloat16, device="cuda")
    x = layer.dev["x"] if T else torch.empty((1, w.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_forward(layer.desc, layer.weights, x, out, counts, ntie, layer.ws)
    torch.cuda.synchronize()
    assert int(counts.sum().item()) == T * w.K and int(ntie.item()) >= 0
    if T:
        ref, _, _, _ = oracle.Oracle(w, a).forward()
        assert max_abs_rel(f64(out), ref) <= TOL["bf16"]


# ------------------------------------------------------------ entry points alone

DISPATCH_CASES = [
    # (T, K, E) ; the page's example first
    (3, 2, 3), (1, 1, 1), (5000, 2, 4), (4096 * 3 // 8 + 37, 8, 64), (700, 3, 1000),
    (2049, 8, 256), (2048, 8, 256), (9000, 2, 16),
    # one workgroup: every round of 1024 slots, the most experts, ragged ends
    (16383, 1, 256), (4097, 4, 200), (1025, 1, 2),
    # one workgroup, few rounds of 1024 slots, few and many experts
    (700, 2, 128), (2048, 2, 64), (3000, 1, 5), (64, 8, 256),
    # one workgroup, at most 4 experts (one packed scan): up to 16384 slots
    (16384, 1, 4), (8192, 2, 3), (2048, 2, 4), (1, 2, 2), (333, 4, 4), (5461, 3, 4),
    # just past one workgroup, few experts: the three-launch path
    (8193, 2, 4),
    # 2^21 slots and more: the scan over unpacked counts (scan_kernel)
    (262144, 8, 64), (262147, 8, 64), (1 << 21, 1, 256),
]


@pytest.mark.parametrize("T,K,E", DISPATCH_CASES)
def test_dispatch_matches_counting_sort(T, K, E):
    """moe_dispatch fed the ids: counts, offsets, perm, sorted_token, inv,
    sorted_w bit-exact, rows_sorted a bitwise gather (StableLatentMoE
    'Dispatch is a stable permutation')."""
    say(f"case dispatch T={T} K={K} E={E}")
    rng = np.random.default_rng(T + 7 * E)
    if (T, K, E) == (3, 2, 3):
        idx = np.array([[2, 0], [0, 2], [2, 1]], np.int32)
    elif T * K >= 1 << 20 and K == 1:
        idx = rng.integers(0, E, size=(T, 1), dtype=np.int32)
    elif T * K >= 1 << 20:  # K distinct experts per token, drawn in one pass
        idx = np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :K].astype(np.int32)
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    g = rng.random((T, K)).astype(np.float32)
    w = custom(name="disp", T=T, K=K, E=E, d=16, act="bf16")
    rows = moe_synth.draw_rows(77 + T, (T, w.d), "bf16")
    desc = moe.make_desc(w)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    d_idx, d_g = cu(idx), cu(g)
    d_rows = cu(rows.view(np.int16))
    n = T * K
    i32 = lambda m: torch.full((m,), -9, dtype=torch.int32, device="cuda")
    counts, offsets, perm, st, inv = i32(E), i32(E + 1), i32(n), i32(n), i32(n)
    sw = torch.full((n,), -9.0, dtype=torch.float32, device="cuda")
    rs = torch.zeros((n, w.d), dtype=torch.int16, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(desc), dtype=torch.uint8, device="cuda")
    moe.moe_dispatch(desc, d_idx, d_g, d_rows, counts, offsets, perm, st, inv, sw, rs, ws)
    torch.cuda.synchronize()
    r = oracle.dispatch(idx, g, E)
    for k in ("counts", "offsets", "perm", "sorted_token", "inv"):
        got = {"counts": counts, "offsets": offsets, "perm": perm, "sorted_token": st,
               "inv": inv}[k].cpu().numpy()
        assert np.array_equal(got, r[k]), k
    assert np.array_equal(sw.cpu().numpy(), r["sorted_w"])
    assert np.array_equal(rs.cpu().numpy().view(np.uint16), rows[r["sorted_token"]])


@pytest.mark.parametrize("name,kw", [
    ("tiny", None), ("small", None),
    ("ragged_bf16", EDGE["ragged_bf16"]), ("latent_f32", EDGE["latent_f32"]),
    ("skewed", dict(T=400, d=64, d_ff=48, E=16, K=2, act="bf16")),
])
@pytest.mark.parametrize("fused_gather", [True, False])
def test_expert_ffn_alone(name, kw, fused_gather):
    """moe_expert_ffn on the oracle's dispatch: y_sorted[p] = sorted_w[p] *
    FFN_e(row) for every sorted row (Math. Reference 12.2)."""
    w = moe_synth.get(name) if kw is None else custom(name=name, **kw)
    say(f"case expert_ffn {name} fused_gather={fused_gather}")
    a = moe_synth.generate(w)
    orc = oracle.Oracle(w, a)
    idx, g, _, _ = orc.route()
    if name == "skewed":
        idx[: w.T * 3 // 4, 0] = 0  # most tokens on expert 0 in slot 0
        idx[:, 1] = np.where(idx[:, 1] == 0, 1, idx[:, 1])
    r = oracle.dispatch(idx, g.astype(np.float32), w.E)
    de = w.d_e
    src = a["x"] if not w.latent else moe_synth.draw_rows(91, (w.T, de), w.act)
    expert_of = np.repeat(np.arange(w.E), r["counts"]).astype(np.int32)
    ref = orc.expert_rows(src[r["sorted_token"]], expert_of, r["sorted_w"])
    dev = dev_of(a)
    layer = layer_of(w, a, dev)
    cu = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    act_t = torch.bfloat16 if w.act == "bf16" else torch.float32
    def dev_rows(x):
        t = cu(x)
        return t.view(torch.bfloat16) if x.dtype == np.uint16 else t
    rows_t = dev_rows(src if fused_gather else src[r["sorted_token"]])
    ri = cu(r["sorted_token"]) if fused_gather else None
    y = torch.full((w.T * w.K, de), float("nan"), dtype=act_t, device="cuda")
    moe.moe_expert_ffn(layer.desc, layer.weights, rows_t, ri, cu(r["offsets"]),
                       cu(r["sorted_w"]), y, layer.ws)
    torch.cuda.synchronize()
    err = max_abs_rel(f64(y), ref)
    say(f"  expert_ffn max-abs-rel {err:.3e}")
    assert err <= TOL[w.act]


@pytest.mark.parametrize("name,kw", [
    ("tiny", None), ("small", None), ("no_shared_bf16", EDGE["no_shared_bf16"]),
    ("latent_f32", EDGE["latent_f32"]), ("latent_bf16_noshared", EDGE["latent_bf16_noshared"]),
])
def test_combine_alone(name, kw):
    """moe_combine on stand-in routed rows: out[t] = shared(x_t) + sum_k
    y[inv[t*K+k]] (latent: W_lat_up RMSNorm(.)) (Math. Reference 13.2)."""
    w = moe_synth.get(name) if kw is None else custom(name=name, **kw)
    say(f"case combine {name}")
    a = moe_synth.generate(w)
    orc = oracle.Oracle(w, a)
    idx, g, _, _ = orc.route()
    r = oracle.dispatch(idx, g.astype(np.float32), w.E)
    y = moe_synth.draw_rows(313, (w.T * w.K, w.d_e), w.act, std=0.1)
    ref = orc.combine(y, r["inv"])
    layer = layer_of(w, a)
    yt = torch.from_numpy(y).cuda()
    if y.dtype == np.uint16:
        yt = yt.view(torch.bfloat16)
    inv = torch.from_numpy(r["inv"]).cuda()
    out = torch.empty((w.T, w.d), dtype=yt.dtype, device="cuda")
    moe.moe_combine(layer.desc, layer.weights, layer.dev["x"], yt, inv, out, layer.ws)
    torch.cuda.synchronize()
    err = max_abs_rel(f64(out), ref)
    say(f"  combine max-abs-rel {err:.3e}")
    assert err <= TOL[w.act]


def test_forward_is_deterministic():
    """No atomics in the combine: two runs give the same bytes."""
    w = custom(name="det", T=500, d=64, d_ff=64, E=8, K=3, act="bf16")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    say("case determinism")
    o1 = layer.forward(layer.dev["x"]).clone()
    o2 = layer.forward(layer.dev["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_side_stream_forward_matches_single_stream():
    """A layer large enough for 256x256 tiles with shared experts runs the
    shared gate/up GEMM on a second stream beside routing and the routed
    GEMMs; with a timing probe everything runs on the caller's stream. Both
    must give the same bytes, repeatably, and match the oracle."""
    w = custom(name="side", config_no=931, T=4096, d=1024, d_ff=1024, E=8, K=2, act="bf16",
               n_shared=1, d_ff_shared=1024, w_std=0.03, router_std=0.03, bias_std=0.01)
    plan = moe.moe_plan(moe.make_desc(w))
    assert plan["merged_shared"] == 0 and plan["gate_up_tile_m"] == 256
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    say("case side stream")
    x = layer.dev["x"]
    o1 = layer.forward(x).clone()
    o2 = layer.forward(x).clone()
    probe = moe.MoeProbe(stage=-1, repeat=1, ev_begin=None, ev_end=None)
    o3 = layer.forward(x, probe=probe).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    check_forward(w, a, layer, tokens=np.arange(0, w.T, 7))


def test_probe_records_stage_events():
    w = moe_synth.get("tiny")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    b = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    b.record()
    e.record()  # creates the events on the current stream
    torch.cuda.synchronize()
    probe = moe.MoeProbe(stage=moe.STAGES["expert_gate_up"], ev_begin=b.cuda_event,
                         ev_end=e.cuda_event)
    layer.forward(layer.dev["x"], probe=probe)
    torch.cuda.synchronize()
    assert b.elapsed_time(e) > 0


@pytest.mark.parametrize("stage,merged", [("expert_gate_up", 1), ("expert_down", 1),
                                          ("expert_gate_up", 0), ("shared_gate_up", 0)])
def test_probe_repeat_keeps_the_result(stage, merged):
    """Repeated passes of a GEMM stage (timing aid) leave the output bitwise
    unchanged, with the shared experts merged into the grouped launches
    (small layer) or not (an expert width the pipelined kernel does not
    take)."""
    w = moe_synth.get("small").with_T(512) if merged else custom(
        "probe_sep", T=300, d=64, d_ff=40, E=4, K=2, act="bf16", n_shared=1, d_ff_shared=64)
    assert moe.moe_plan(moe.make_desc(w))["merged_shared"] == merged
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    ref = layer.forward(layer.dev["x"]).clone()
    b = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    b.record()
    e.record()
    torch.cuda.synchronize()
    probe = moe.MoeProbe(stage=moe.STAGES[stage], repeat=7, ev_begin=b.cuda_event,
                         ev_end=e.cuda_event)
    out = layer.forward(layer.dev["x"], probe=probe)
    torch.cuda.synchronize()
    assert b.elapsed_time(e) > 0
    assert torch.equal(out, ref)


# ---------------------------------------------------------------- balancer
def _balance_gpu(E, K, N, counts, bias, alpha):
    c = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int32)).cuda()
    b = torch.from_numpy(np.array(bias, dtype=np.float32)).cuda()
    moe.moe_balance_bias(E, K, N, c, alpha, b)
    torch.cuda.synchronize()
    return b.cpu().numpy()


def test_balance_bias_worked_example():
    """Part 3, section 14.5 on the device: [0]*4 -> [-0.1, 0, 0.1, 0]."""
    say("case balance worked example")
    out = _balance_gpu(4, 2, 8, [5, 4, 3, 4], [0, 0, 0, 0], 0.1)
    assert np.array_equal(out, oracle.balance_bias([5, 4, 3, 4], [0, 0, 0, 0], 0.1, 8, 2))
    assert np.array_equal(out, np.float32([-0.1, 0.0, 0.1, 0.0]))


@pytest.mark.parametrize("E,K,N,seed", [(4, 2, 2048, 0), (64, 8, 8192, 1), (256, 8, 16384, 2),
                                        (1024, 2, 40, 3), (300, 7, 977, 4), (1, 1, 5, 5)])
def test_balance_bias_matches_oracle(E, K, N, seed):
    """Bit-exact against the oracle on random loads, biases beyond the clamp
    range included; a third of the experts are set exactly balanced."""
    say(f"case balance E={E} K={K} N={N} seed={seed}")
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(N * K, np.ones(E) / E).astype(np.int32)
    if (N * K) % E == 0:
        counts[: E // 3] = (N * K) // E
    bias = rng.uniform(-1.3, 1.3, E).astype(np.float32)
    alpha = float(np.float32(rng.uniform(0.001, 0.3)))
    got = _balance_gpu(E, K, N, counts, bias, alpha)
    want = oracle.balance_bias(counts, bias, alpha, N, K)
    assert np.array_equal(got, want)


def test_balance_bias_exact_at_large_token_counts():
    """N K = 2^30 with E = 256: an expert off by one assignment must still
    move (1/E - c/(N K) = 2^-30, below fp32 resolution of 1/E), a balanced
    one must not."""
    say("case balance large N")
    E, K, N = 256, 8, 2 ** 27
    counts = np.full(E, N * K // E, dtype=np.int32)
    counts[0] += 1
    counts[1] -= 1
    got = _balance_gpu(E, K, N, counts, np.zeros(E, np.float32), 0.01)
    assert got[0] == np.float32(-0.01) and got[1] == np.float32(0.01)
    assert np.all(got[2:] == 0)
    assert np.array_equal(got, oracle.balance_bias(counts, np.zeros(E), 0.01, N, K))


def test_balance_bias_after_forward():
    """The balancer consumes the loads moe_forward returns; the bias it
    writes is the one the next forward's router adds."""
    w = moe_synth.get("small")
    say("case balance after forward small")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    counts = torch.zeros(w.E, dtype=torch.int32, device="cuda")
    layer.forward(layer.dev["x"], counts=counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert int(c.sum()) == w.T * w.K
    b0 = layer.dev["bias"].cpu().numpy().copy()
    moe.moe_balance_bias(w.E, w.K, w.T, counts, 0.05, layer.dev["bias"])
    torch.cuda.synchronize()
    assert np.array_equal(layer.dev["bias"].cpu().numpy(),
                          oracle.balance_bias(c, b0, 0.05, w.T, w.K))


# ---------------------------------------------------------------- QuantileBalancer
QB_TOL = 2e-5  # absolute, on biases of order 0.1: fp32 router and scores vs fp64


@pytest.mark.parametrize("name", ["sigmoid", "sigmoid_renorm_scaled", "latent_f32",
                                  "latent_bf16_noshared", "qb_e1024", "qb_one_token"])
def test_quantile_balance_matches_oracle(name):
    extra = {"qb_e1024": dict(T=300, d=32, d_ff=8, E=1024, K=8, route="sigmoid_bias",
                              bias_std=0.05, act="bf16"),
             "qb_one_token": dict(T=1, E=9, K=3, route="sigmoid_bias", bias_std=0.1)}
    w = custom(name, **(EDGE.get(name) or extra[name]))
    say(f"case quantile_balance {name} T={w.T} E={w.E} K={w.K} act={w.act}")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    nb = torch.full((w.E,), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_quantile_balance(layer.desc, layer.weights, layer.dev["x"], nb, layer.ws)
    torch.cuda.synchronize()
    got = nb.cpu().numpy().astype(np.float64)
    want = oracle.Oracle(w, a).quantile_balance()
    err = float(np.max(np.abs(got - want)))
    say(f"  max abs err {err:.2e}, sum {got.sum():.2e}")
    assert err <= QB_TOL
    assert abs(got.sum()) <= 1e-5 * w.E


def test_quantile_balance_in_place_replaces_the_buffer():
    """new_bias may be the layer's own bias (the page copies into the
    buffer): same result as writing elsewhere, and the next route uses it."""
    w = custom("qb_inplace", **EDGE["sigmoid"])
    say("case quantile_balance in place")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    other = torch.empty(w.E, dtype=torch.float32, device="cuda")
    moe.moe_quantile_balance(layer.desc, layer.weights, layer.dev["x"], other, layer.ws)
    moe.moe_quantile_balance(layer.desc, layer.weights, layer.dev["x"], layer.dev["bias"], layer.ws)
    torch.cuda.synchronize()
    assert torch.equal(other, layer.dev["bias"])
    a2 = dict(a)
    a2["bias"] = layer.dev["bias"].cpu().numpy()
    check_route(w, a2, layer)


# ---------------------------------------------------------------- router losses
LOSS_RTOL = 1e-5  # fp32 logits and per-token softmax vs fp64


def _router_losses_gpu(layer, counts, alpha, z_weight):
    losses = torch.full((2,), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_losses(layer.desc, layer.weights, layer.dev["x"], counts, alpha, z_weight,
                          losses, layer.ws)
    torch.cuda.synchronize()
    return losses.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["tiny", "small", "sigmoid", "e1024", "k16", "many_chunks",
                                  "valu_wide", "split_router"])
def test_router_losses_match_oracle(name):
    """Switch load-balancing loss (moe-from-scratch page) and router z-loss
    (transformer book page) on the loads the forward returned, against the
    oracle on the same loads; valu_wide is the widest model of the
    wavefront-per-token router, split_router has few tokens and a wider
    model, so the matrix-core router GEMM splits its reduction."""
    extra = {"valu_wide": dict(T=100, d=2048, d_ff=16, E=64, K=8, act="bf16",
                               router_std=0.02, w_std=0.02),
             "split_router": dict(T=100, d=2560, d_ff=16, E=64, K=8, act="bf16",
                                  router_std=0.02, w_std=0.02)}
    if name in ("tiny", "small"):
        w = moe_synth.get(name)
    else:
        w = custom(name, config_no=700 + len(name), **(EDGE.get(name) or extra[name]))
    say(f"case router_losses {name} T={w.T} d={w.d} E={w.E} K={w.K} act={w.act}")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    layer.forward(layer.dev["x"], counts=counts)
    got = _router_losses_gpu(layer, counts, 0.01, 0.001)
    want = np.array(oracle.Oracle(w, a).router_losses(counts.cpu().numpy(), 0.01, 0.001))
    rel = np.abs(got - want) / np.abs(want)
    say(f"  losses gpu {got} oracle {want} rel {rel}")
    assert np.all(rel <= LOSS_RTOL)


def test_router_losses_uniform_router_and_determinism():
    """Zero router weights: every softmax is uniform, so with equal loads
    the Switch loss is alpha exactly and the z-loss z_weight (log E)^2; two
    calls give the same bits; T = 0 leaves the output untouched."""
    w = custom("loss_uniform", T=256, E=8, K=2, act="bf16", router_std=0.0, bias_std=0.0)
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    counts = torch.full((w.E,), w.T * w.K // w.E, dtype=torch.int32, device="cuda")
    got = _router_losses_gpu(layer, counts, 0.01, 0.001)
    assert abs(got[0] - 0.01) <= 1e-7
    assert abs(got[1] - 0.001 * np.log(w.E) ** 2) <= 1e-8
    assert np.array_equal(got, _router_losses_gpu(layer, counts, 0.01, 0.001))
    d0 = moe.make_desc(w.with_T(0))
    keep = torch.full((2,), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_router_losses(d0, layer.weights, layer.dev["x"], counts, 0.01, 0.001, keep, layer.ws)
    torch.cuda.synchronize()
    assert keep.tolist() == [7.0, 7.0]
