"""CPU checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes as C
import os
import re

import pytest

import mixture_experts_ffn_fp32_amd as moe
import moe_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]*?\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    # nothing internal leaks out with default visibility
    out = os.popen(f"nm -D --defined-only {moe.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(declared_symbols()) <= exported
    assert not [s for s in exported if "moe" in s and s not in declared_symbols()]


def test_strerror_and_stage_names():
    assert moe.strerror(0) == "ok"
    assert moe.strerror(-4) == "workspace too small"
    assert moe.strerror(12345) == "unknown status"
    assert [moe.stage_name(i) for i in range(7)] == list(moe.STAGES)
    assert moe.stage_name(99) == "?"


def test_struct_layout_matches_header():
    # moe_desc: int64 + 10 int32 + 2 float = 56 bytes; moe_weights: 11 pointers
    assert C.sizeof(moe.MoeDesc) == 56
    assert C.sizeof(moe.MoeWeights) == 11 * 8
    assert C.sizeof(moe.MoeProbe) == 24


def _desc(**kw):
    w = moe_synth.get("small")
    d = moe.make_desc(w)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_workspace_size_scales_with_tokens():
    small = moe.moe_workspace_size(_desc(T=64))
    big = moe.moe_workspace_size(_desc(T=4096))
    assert 0 < small < big
    w = moe_synth.get("large_prefill")
    n = moe.moe_workspace_size(moe.make_desc(w))
    rows = w.T * w.K
    # at least the routed intermediate and outputs (bf16)
    assert n >= rows * (w.d_ff + w.d) * 2
    assert moe.moe_workspace_size(_desc(T=0)) >= 0


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), -2), (dict(d_model=0), -2), (dict(d_model=500), -2), (dict(d_ff=1370), -2),
    (dict(top_k=0), -2), (dict(top_k=5), -2), (dict(n_experts=2000, top_k=2), -2),
    (dict(n_experts=32, top_k=17), -2), (dict(act_dtype=7), -3), (dict(route_mode=3), -3),
    (dict(has_rmsnorm=1), -3), (dict(d_shared=12), -2), (dict(latent=20), -2),
])
def test_bad_descriptors_rejected(kw, status):
    with pytest.raises(moe.MoeError) as e:
        moe.moe_workspace_size(_desc(**kw))
    assert e.value.status == status


def test_null_pointers_rejected_before_launch():
    d = _desc(T=16)
    w = moe.MoeWeights()
    with pytest.raises(moe.MoeError) as e:
        moe.lib() and moe.moe_route(d, w, None, None, None, stream=0)
    assert e.value.status == -1
    rc = moe.lib().moe_forward(C.byref(d), C.byref(w), None, None, None, None, None, 0, None, None)
    assert rc == -1
    rc = moe.lib().moe_dispatch(C.byref(d), None, None, None, None, None, None, None, None, None,
                                None, None, 0, None)
    assert rc == -1


def test_binding_refuses_host_and_strided_tensors():
    """The binding passes device addresses only: a host tensor or a strided
    view is refused before the library is called."""
    import torch
    d = _desc(T=16)
    w = moe.MoeWeights()
    with pytest.raises(ValueError, match="device tensors"):
        moe.moe_route(d, w, torch.zeros(16, 64), None, None, stream=0)
    assert moe._ptr(None) is None

    class _View:  # stands in for a device tensor whose view is strided
        is_cuda = True

        @staticmethod
        def is_contiguous():
            return False

        shape, dtype = (16, 64), torch.bfloat16
    with pytest.raises(ValueError, match="contiguous"):
        moe._ptr(_View())


def test_misaligned_arrays_rejected_before_launch():
    """Activations, weights, outputs, gradients and workspaces must be 16-byte
    aligned; a misaligned one is a shape error found on the host (the fake
    addresses are never dereferenced)."""
    d = _desc(T=16)
    a, bad = 1 << 20, (1 << 20) + 8
    w = moe.MoeWeights(w_router=a, w_gate=a, w_up=a, w_down=a, ws_gate=a, ws_up=a, ws_down=a)
    big = 1 << 40
    rc = moe.lib().moe_route(C.byref(d), C.byref(w), bad, a, a, None, None, a, big, None)
    assert rc == -2
    rc = moe.lib().moe_forward(C.byref(d), C.byref(w), a, bad, None, None, a, big, None, None)
    assert rc == -2
    w_bad = moe.MoeWeights(w_router=a, w_gate=a, w_up=bad, w_down=a, ws_gate=a, ws_up=a,
                           ws_down=a)
    rc = moe.lib().moe_forward(C.byref(d), C.byref(w_bad), a, a, None, None, a, big, None, None)
    assert rc == -2
    g = moe.MoeGrads(w_gate=bad)
    rc = moe.lib().moe_backward(C.byref(d), C.byref(w), a, a, a, C.byref(g), a, big, None)
    assert rc == -2
    # aligned: past these checks, to the workspace size check
    rc = moe.lib().moe_route(C.byref(d), C.byref(w), a, a, a, None, None, a, 16, None)
    assert rc == -4


def test_workspace_too_small_rejected():
    d = _desc(T=16)
    fake = 1 << 20  # never dereferenced: the size check fails first
    rc = moe.lib().moe_dispatch(C.byref(d), fake, fake, None, fake, fake, fake, fake, fake, None,
                                None, fake, 16, None)
    assert rc == -4


@pytest.mark.parametrize("args,status", [
    ((0, 1, 8), -2), ((1025, 1, 8), -2), ((4, 0, 8), -2), ((4, 5, 8), -2), ((4, 2, -1), -2),
    ((4, 2, 2 ** 31), -2),
])
def test_balance_bias_bad_shapes_rejected(args, status):
    """Checked on the host before any launch (no device pointers needed)."""
    dummy = C.c_void_p(16)
    assert moe.lib().moe_balance_bias(*args, dummy, 0.1, dummy, None) == status


def test_balance_bias_null_and_alpha_rejected():
    dummy = C.c_void_p(16)
    assert moe.lib().moe_balance_bias(4, 2, 8, None, 0.1, dummy, None) == -1
    assert moe.lib().moe_balance_bias(4, 2, 8, dummy, 0.1, None, None) == -1
    assert moe.lib().moe_balance_bias(4, 2, 8, dummy, float("nan"), dummy, None) == -3
    assert moe.lib().moe_balance_bias(4, 2, 8, dummy, float("inf"), dummy, None) == -3
    # zero tokens: a no-op that touches nothing
    assert moe.lib().moe_balance_bias(4, 2, 0, dummy, 0.1, dummy, None) == 0


def test_quantile_balance_checked_before_launch():
    """Sigmoid routing with K < E only; NULLs and a short workspace are
    reported before anything is enqueued; the workspace of a sigmoid-routed
    layer holds the balancer's buffers."""
    fake = C.c_void_p(1 << 20)
    w = moe.MoeWeights()
    w.w_router = fake
    sig = _desc(T=16, route_mode=2)
    n_sig = moe.moe_workspace_size(sig)
    assert n_sig > moe.moe_workspace_size(_desc(T=16))
    L = moe.lib()
    assert L.moe_quantile_balance(C.byref(_desc(T=16)), C.byref(w), fake, fake, fake, n_sig,
                                  None) == -3
    assert L.moe_quantile_balance(C.byref(_desc(T=16, route_mode=2, top_k=4)), C.byref(w), fake,
                                  fake, fake, 1 << 30, None) == -2
    assert L.moe_quantile_balance(C.byref(sig), C.byref(w), fake, None, fake, n_sig, None) == -1
    assert L.moe_quantile_balance(C.byref(sig), C.byref(w), fake, fake, fake, n_sig - 1,
                                  None) == -4


def test_router_losses_checked_before_launch():
    """NULLs, non-finite weights and a short workspace are reported before
    anything is enqueued; T = 0 is a no-op."""
    fake = C.c_void_p(1 << 20)
    w = moe.MoeWeights()
    w.w_router = fake
    d = _desc(T=16)
    n = moe.moe_workspace_size(d)
    L = moe.lib()
    assert L.moe_router_losses(C.byref(d), C.byref(w), fake, None, 0.01, 0.001, fake, fake, n,
                               None) == -1
    assert L.moe_router_losses(C.byref(d), C.byref(w), fake, fake, 0.01, 0.001, None, fake, n,
                               None) == -1
    assert L.moe_router_losses(C.byref(d), C.byref(moe.MoeWeights()), fake, fake, 0.01, 0.001,
                               fake, fake, n, None) == -1
    assert L.moe_router_losses(C.byref(d), C.byref(w), fake, fake, float("nan"), 0.001, fake,
                               fake, n, None) == -3
    assert L.moe_router_losses(C.byref(d), C.byref(w), fake, fake, 0.01, float("inf"), fake,
                               fake, n, None) == -3
    assert L.moe_router_losses(C.byref(d), C.byref(w), fake, fake, 0.01, 0.001, fake, fake,
                               n - 1, None) == -4
    d0 = _desc(T=0)
    assert L.moe_router_losses(C.byref(d0), C.byref(w), None, fake, 0.01, 0.001, fake, fake,
                               moe.moe_workspace_size(d0), None) == 0


def test_plan_paths_of_the_workloads():
    """Host-side plan (no GPU): which kernel path and tile each benchmark
    layer takes, so the parity cases can be tied to the paths they cover."""
    P = {n: moe.moe_plan(moe.make_desc(moe_synth.get(n))) for n in
         ("tiny", "small", "medium", "large_prefill", "large_decode", "latent")}
    assert P["small"]["merged_shared"] == 1 and P["small"]["gate_up_pipelined"] == 1
    assert P["small"]["router_per_token"] == 1 and P["small"]["dispatch_one_workgroup"] == 1
    for n in ("medium", "large_prefill", "latent"):
        assert P[n]["merged_shared"] == 0
        assert (P[n]["gate_up_tile_m"], P[n]["gate_up_tile_n"]) == (256, 256)
        assert P[n]["router_per_token"] == 0 and P[n]["dispatch_one_workgroup"] == 0
    assert P["tiny"]["gate_up_pipelined"] == 0  # fp32: generic kernel
    assert (P["large_decode"]["gate_up_tile_m"], P["large_decode"]["gate_up_tile_n"]) == (32, 256)
    assert P["large_decode"]["merged_shared"] == 1
    assert P["large_decode"]["dispatch_one_workgroup"] == 1
    # backward: bf16 expert weights read in place wherever the pipelined
    # kernel takes them (W_down: dh, value 1; W_gate | W_up as two K segments:
    # dX, value 2, needs d_ff a multiple of 64); fp32 layers use copies
    for n in ("large_prefill", "large_decode", "medium", "latent"):
        assert P[n]["backward_in_place"] == 3, n
    assert P["small"]["backward_in_place"] == 1  # d_ff = 1376: dX from copies
    assert P["tiny"]["backward_in_place"] == 0
    # grouped GEMMs on the persistent kernel: 256x256 tiles, two or more per CU
    for n in ("medium", "large_prefill", "latent"):
        assert P[n]["persistent"] == 3, n
    for n in ("tiny", "small", "large_decode"):
        assert P[n]["persistent"] == 0, n
    with pytest.raises(moe.MoeError):
        moe.moe_plan(_desc(T=-1))


@pytest.mark.parametrize("kw, want", [
    # both grouped GEMMs: 256x256 tiles, >= 5 stages, >= 2 tiles per CU
    (dict(T=8229, d=2080, d_ff=1056, E=8, K=4, n_shared=1, d_ff_shared=2048), 3),
    # gate/up reduction of 4 stages (d = 256): only the down GEMM
    (dict(T=65536, d=256, d_ff=2048, E=8, K=2, n_shared=0, d_ff_shared=0), 2),
    # 256x256 gate/up tiles, but fewer than two per CU: neither
    (dict(T=1024, d=2048, d_ff=2048, E=8, K=4, n_shared=0, d_ff_shared=0), 0),
])
def test_plan_persistent_thresholds(kw, want):
    """Host-side plan: which grouped GEMMs take the persistent kernel at the
    edges of its conditions."""
    from _layers import custom
    p = moe.moe_plan(moe.make_desc(custom(name="plan", act="bf16", **kw)))
    assert (p["gate_up_tile_m"], p["gate_up_tile_n"]) == (256, 256)
    assert p["persistent"] == want


def test_backward_checked_before_launch():
    """moe_backward: widths that are multiples of 32; NULLs and a short
    workspace are reported before anything runs."""
    fake = C.c_void_p(1 << 20)
    w = moe.MoeWeights(**{k: fake.value for k, _ in moe.MoeWeights._fields_})
    g = moe.MoeGrads()
    L = moe.lib()
    d = _desc(T=64)
    n = moe.moe_backward_workspace_size(d)
    assert n > moe.moe_workspace_size(d)
    dl = moe.make_desc(moe_synth.get("latent"))
    dl.latent = 40  # latent widths must be multiples of 32 as well
    assert L.moe_backward(C.byref(dl), C.byref(w), fake, fake, fake, C.byref(g), fake, 1 << 40,
                          None) == -2
    assert L.moe_backward(C.byref(_desc(T=64, d_model=520)), C.byref(w), fake, fake, fake,
                          C.byref(g), fake, 1 << 40, None) == -2
    assert L.moe_backward(C.byref(d), C.byref(w), fake, fake, fake, None, fake, n, None) == -1
    assert L.moe_backward(C.byref(d), C.byref(w), None, fake, fake, C.byref(g), fake, n,
                          None) == -1
    assert L.moe_backward(C.byref(d), C.byref(w), fake, fake, fake, C.byref(g), fake, n - 1,
                          None) == -4
    d0 = _desc(T=0)
    assert L.moe_backward(C.byref(d0), C.byref(w), None, None, None, C.byref(g), fake,
                          moe.moe_backward_workspace_size(d0), None) == 0


def test_noalloc_rejects_layers_beyond_the_static_scratch():
    """moe_forward_noalloc checks the layer's workspace against the static
    scratch on the host, before touching any device."""
    fake = C.c_void_p(1 << 20)
    w = moe.MoeWeights(**{k: fake.value for k, _ in moe.MoeWeights._fields_})
    for name in ("medium", "large_prefill", "latent"):
        d = moe.make_desc(moe_synth.get(name))
        assert moe.moe_workspace_size(d) > moe.SCRATCH_BYTES
        assert moe.lib().moe_forward_noalloc(C.byref(d), C.byref(w), fake, fake, None, None,
                                             None) == -6
    for name, T in (("small", 2048), ("large_decode", 256), ("tiny", 128)):
        d = moe.make_desc(moe_synth.get(name).with_T(T))
        assert moe.moe_workspace_size(d) <= moe.SCRATCH_BYTES
    assert "static scratch" in moe.strerror(-6)
