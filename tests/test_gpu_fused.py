"""Parity of one-token layers whose down projection and combine run as one
kernel (H=2048 with a shared expert, row and affine formats) through the C
ABI: forward, residual form and a missing expert."""
import numpy as np
import pytest

import oracle
import synth
from parity import OracleLayer, check_ids, flags, log, rel_err, REL_TOL, check_residual

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M  # noqa: E402
from int4_weight_expert_amd import workload  # noqa: E402

NAMES = ["mid_row", "mid_affine"]


@pytest.fixture(scope="module", params=NAMES)
def case(request):
    cfg = synth.CONFIGS[request.param]
    ml = workload.build_layer(cfg, max_tokens=4)
    yield cfg, ml, OracleLayer(cfg, 0)
    ml.close()


@pytest.mark.parametrize("stream", [0, 1, 2])
def test_forward_matches_oracle(case, stream):
    cfg, layer, ref = case
    log(f"{cfg.name} forward T=1 stream={stream}")
    x = synth.tokens(cfg, T=1, stream=stream)
    out = layer.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
    ids, w = layer.route(torch.from_numpy(x).cuda(), 0)
    rc, missing = layer.status()
    assert rc == 0, missing
    r_out, r_ids, r_w, gk, gi = ref.forward(x)
    check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, cfg.name)
    excluded, _ = flags(gk, gi)
    err = rel_err(out, r_out, ~excluded)
    log(f"  max|d|/max|ref| = {err:.3e}")
    assert err <= REL_TOL


def test_residual_matches_oracle(case):
    cfg, layer, ref = case
    x = synth.tokens(cfg, T=1, stream=50) * 3.0
    xd = torch.from_numpy(x).cuda()
    layer.forward_residual(xd, 0)
    r_out, _, _, gk, gi = ref.forward(x, residual=True)
    excluded, _ = flags(gk, gi)
    e_next, e_term = check_residual(x, xd.cpu().numpy(), r_out, ~excluded, cfg.name)
    log(f"{cfg.name} residual: max|d|/max|ref| = {e_next:.3e} (new x), {e_term:.3e} (moe term)")


def test_missing_expert_contributes_nothing(case):
    cfg, layer, ref = case
    x = synth.tokens(cfg, T=1, stream=60)
    _, r_ids, r_w, _, _ = ref.forward(x)
    victim = int(r_ids[0, 1])
    layer.map(0, victim, -1)
    try:
        out = layer.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
        rc, missing = layer.status()
        assert rc == M.MOE_E_NOT_RESIDENT and missing == [victim]
        ref.need(r_ids)
        acc = np.zeros(cfg.H)
        for s in range(cfg.n_shared):
            acc += oracle.expert(cfg.fmt, cfg.H, cfg.I, ref.shared[s], x[0])[0]
        for k in range(cfg.K):
            e = int(r_ids[0, k])
            if e != victim:
                acc += float(r_w[0, k]) * oracle.expert(cfg.fmt, cfg.H, cfg.I, ref.cache[e], x[0])[0]
        err = rel_err(out[0], acc)
        log(f"{cfg.name} missing expert {victim}: max|d|/max|ref| = {err:.3e}")
        assert err <= REL_TOL
    finally:
        layer.map(0, victim, victim)
