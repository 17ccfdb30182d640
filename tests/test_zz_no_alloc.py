"""moe_set_router_noalloc (the router setter for callers that cannot
allocate device memory) against moe_set_router, through the C ABI: two
calls in a row on one device, the second with a smaller router (the fixed
staging array keeps the first call's larger contents), each checked by the
routing and the layer outputs it produces, which must equal bit for bit
those of the same router set by moe_set_router."""
import numpy as np
import pytest

import synth
from parity import OracleLayer, check_ids, flags, log, rel_err, REL_TOL
from synth.configs import LayerConfig, W_INT4_ROW

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M, workload  # noqa: E402


def _case(name, H, I, E, K, seed):
    return LayerConfig(name=name, H=H, I=I, E=E, K=K, n_shared=1, fmt=W_INT4_ROW, T=4,
                       n_layers=1, seed=seed, zipf_c=0.2)


def _check_pair(cfg, host_source: bool):
    """Layer 0's router set by moe_set_router, layer 1's (the same weights)
    by moe_set_router_noalloc; layer 1 maps the same expert slots and holds
    the same shared expert."""
    ml = workload.build_layer(cfg.with_(n_layers=2), max_tokens=16)
    try:
        W, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
        ml.set_router(0, W, b)
        src = W if host_source else torch.from_numpy(W).cuda()
        bsrc = b if host_source else torch.from_numpy(b).cuda()
        M._check("moe_set_router_noalloc", M.moe_set_router_noalloc(ml.ctx, 1, src, bsrc))
        for e in range(cfg.E):
            ml.map(1, e, e)           # layer 1 reads layer 0's expert slots
        ml.set_shared(1, 0, ml.read_shared(0, 0))   # and layer 0's shared expert
        ref = OracleLayer(cfg, 0)
        for T in (1, 5, 16):
            x = torch.from_numpy(synth.tokens(cfg, T=T, stream=T)).cuda()
            ids0, w0 = ml.route(x, 0)
            ids1, w1 = ml.route(x, 1)
            assert torch.equal(ids0, ids1) and torch.equal(w0.view(torch.int32),
                                                           w1.view(torch.int32)), T
            o0 = ml.forward(x, 0).clone()
            o1 = ml.forward(x, 1).clone()
            assert torch.equal(o0.view(torch.int32), o1.view(torch.int32)), T
            r_out, r_ids, r_w, gk, gi = ref.forward(x.cpu().numpy())
            check_ids(ids1.cpu().numpy(), r_ids, w1.cpu().numpy(), r_w, gk, gi, f"{cfg.name} T={T}")
            excluded, _ = flags(gk, gi)
            err = rel_err(o1.cpu().numpy(), r_out, ~excluded)
            log(f"{cfg.name} T={T}: noalloc router equals moe_set_router bit for bit; "
                f"max|d|/max|ref| = {err:.2e}")
            assert err <= REL_TOL
        assert ml.status()[0] == M.MOE_OK
        assert M.moe_set_router_noalloc(ml.ctx, 2, src, bsrc) == M.MOE_E_ARG
        assert M.moe_set_router_noalloc(ml.ctx, 0, None, bsrc) == M.MOE_E_ARG
    finally:
        ml.close()


def test_noalloc_router_two_calls_second_smaller():
    # first call: 256 experts x 6144 inputs (the GLM router, 6.3 MB staged)
    _check_pair(_case("noalloc_big", 6144, 256, 256, 8, 960), host_source=False)
    # second call: 32 experts x 512 inputs, from host memory
    _check_pair(_case("noalloc_small", 512, 256, 32, 4, 961), host_source=True)
