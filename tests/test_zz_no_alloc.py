"""moe_layer_noalloc (the layer on the library's static device scratch, for
callers that cannot allocate) against moe_layer with a caller workspace: two
calls in a row per case, the second on a smaller batch, each bit-identical
to moe_layer's output and routing (the same kernels run on the same inputs;
the scratch keeps the previous call's contents, which no kernel reads)."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import config, device_inputs, host, norm_err
from oracle import ffn, formats

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("block_scaled_fp4_sqrtsoftplus_amd")


def _both(wl, d, T):
    cfg = config(moe, wl, tokens=T)
    x = d["x"][:T].contiguous()
    ids = d["token_ids"][:T].contiguous()
    y_ref, r_ref = moe.layer(cfg, x, d["weights"], w_gate=d["w_gate"], bias=d["bias"], token_ids=ids,
                             shared=d["shared"], want_routing=True)
    y = torch.empty_like(y_ref)
    r = moe._routing_tensors(T, wl.top_k, wl.n_experts, x.device)
    moe.layer_noalloc(cfg, x, d["weights"], y, w_gate=d["w_gate"], bias=d["bias"], token_ids=ids,
                      shared=d["shared"], routing=r)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"T={T}: y differs"
    for k in r_ref:
        assert torch.equal(r[k], r_ref[k]), f"T={T}: {k} differs"
    return host(y)


@pytest.mark.parametrize("name,T1,T2,over", [
    # decode shape: the shared expert rides in the routing launches
    ("decode", 64, 19, {}),
    # a shared expert moe_layer forks onto its side stream runs in order here
    ("decode", 48, 7, dict(hidden=1024, inter=512, n_experts=8, top_k=2, shared=True)),
    # 300 tokens: the multi-kernel permutation, the large-batch router
    ("decode", 300, 129, dict(hidden=1024, inter=1024, n_experts=16, top_k=4, shared=True)),
    # hash routing
    ("tiny", 40, 9, dict(mode="hash", n_experts=20, top_k=6, hidden=384, inter=256, shared=True)),
])
def test_noalloc_matches_layer(name, T1, T2, over):
    wl = synth.WORKLOADS[name].replace(**over)
    print(f"[noalloc] {name} {over} T={T1} then T={T2}", flush=True)
    inp = synth.make_inputs(wl, tokens=T1)
    d = device_inputs(inp)
    y1 = _both(wl, d, T1)
    _both(wl, d, T2)
    if wl.hidden <= 1024:
        # the first call also against the oracle
        ref = ffn.layer(inp, wl.top_k, wl.route_scale, wl.swiglu_limit, wl.mode, wl.seed)
        err = norm_err(formats.bf16_decode(y1), ref["y"])
        print(f"[noalloc] vs oracle {err:.2e}")
        assert err <= 2e-2

