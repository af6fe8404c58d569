"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration the benchmark times: routing and dispatch on every token,
layer outputs on a seeded token sample the oracle evaluates one by one."""
import numpy as np
import pytest

import mixture_experts_ffn_fp32_amd as moe
import moe_synth
import oracle
from _gpu import check_forward, check_route, layer_of, need_gpu, sample_tokens, say, torch

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

SAMPLE = {"medium": 1024, "latent": 1024, "large_decode": None, "large_prefill": 1024}


@pytest.mark.parametrize("name", ["medium", "latent", "large_decode", "large_prefill"])
def test_full_size_workload(name):
    need_gpu()
    w = moe_synth.get(name)
    say(f"case full {name}: generating inputs")
    a = moe_synth.generate(w)
    layer = layer_of(w, a)
    orc = oracle.Oracle(w, a)
    say(f"  {name}: route (all {w.T} tokens)")
    r = check_route(w, a, layer, orc)
    o_idx = r[0]
    n = SAMPLE[name]
    toks = None if n is None else sample_tokens(o_idx, w.E, n, seed=w.config_no)
    say(f"  {name}: forward")
    check_forward(w, a, layer, tokens=toks, orc=orc, o_route=r)
    if name == "medium":
        counts = np.bincount(o_idx.ravel(), minlength=w.E)
        assert (counts == 0).sum() == moe_synth.ZIPF_EMPTY
        say("  medium: router losses (skewed loads)")
        c = torch.tensor(counts, dtype=torch.int32, device="cuda")
        losses = torch.empty(2, dtype=torch.float32, device="cuda")
        moe.moe_router_losses(layer.desc, layer.weights, layer.dev["x"], c, 0.01, 0.001, losses,
                              layer.ws)
        torch.cuda.synchronize()
        got = losses.cpu().numpy().astype(np.float64)
        want = np.array(orc.router_losses(counts, 0.01, 0.001))
        say(f"  medium: losses {got} oracle {want}")
        assert np.all(np.abs(got - want) <= 1e-5 * np.abs(want))
    if name == "latent":  # QuantileBalancer update over all tokens
        say("  latent: quantile balance")
        nb = torch.empty(w.E, dtype=torch.float32, device="cuda")
        moe.moe_quantile_balance(layer.desc, layer.weights, layer.dev["x"], nb, layer.ws)
        torch.cuda.synchronize()
        err = float(np.max(np.abs(nb.cpu().numpy() - orc.quantile_balance())))
        say(f"  latent: quantile balance max abs err {err:.2e}")
        assert err <= 2e-5
    del layer, a
    torch.cuda.empty_cache()
