"""moe_forward_noalloc (the forward in the library's static device scratch,
for callers that cannot allocate) against moe_forward on the same layers:
calls in a row on one GPU, each later one smaller than the one before, so
the scratch holds the previous call's contents; outputs, loads and
near-tie counts must be identical to moe_forward's."""
import numpy as np
import pytest

import mixture_experts_ffn_fp32_amd as moe
import moe_synth
from _gpu import layer_of, need_gpu, say, torch

pytestmark = pytest.mark.gpu


def _run(layer, noalloc):
    w = layer.spec
    out = torch.full((w.T, w.d), float("nan"), dtype=layer.act, device="cuda")
    counts = torch.full((w.E,), -1, dtype=torch.int32, device="cuda")
    ntie = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    if noalloc:
        moe.moe_forward_noalloc(layer.desc, layer.weights, layer.dev["x"], out, counts, ntie)
    else:
        moe.moe_forward(layer.desc, layer.weights, layer.dev["x"], out, counts, ntie, layer.ws)
    torch.cuda.synchronize()
    return out.cpu(), counts.cpu(), ntie.cpu()


def test_noalloc_matches_forward_on_consecutive_calls():
    need_gpu()
    cases = [("small", 2048), ("small", 300), ("tiny", 128), ("tiny", 37)]
    for name, T in cases:
        w = moe_synth.get(name).with_T(T)
        assert moe.moe_workspace_size(moe.make_desc(w)) <= moe.SCRATCH_BYTES
        say(f"case noalloc {name} T={T}")
        layer = layer_of(w, moe_synth.generate(w))
        got = _run(layer, True)
        want = _run(layer, False)
        for g, e, what in zip(got, want, ("out", "counts", "n_near_ties")):
            assert torch.equal(g.view(torch.int16) if g.dtype == torch.bfloat16 else g,
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e), what
        assert int(got[1].sum()) == w.T * w.K
        assert not torch.isnan(got[0].float()).any()
        say(f"  noalloc {name} T={T}: identical to moe_forward")
