"""Parity of group-limited routing (8 groups of 32 experts, 4 kept) through the
C ABI: the small-T router tail (T <= 8), the large-T top-k with the GEMV path
(T = 20) and with the grouped GEMM (T = 64, 200), row and affine formats."""
import numpy as np
import pytest

import oracle
import synth
from parity import OracleLayer, check_ids, flags, log, rel_err, REL_TOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import workload  # noqa: E402

TMAX = 200


@pytest.fixture(scope="module", params=["grouped_row", "grouped_affine"])
def case(request):
    cfg = synth.CONFIGS[request.param]
    ml = workload.build_layer(cfg, max_tokens=TMAX)
    yield cfg, ml, OracleLayer(cfg, 0)
    ml.close()


@pytest.mark.parametrize("T", [1, 3, 8, 20, 64, TMAX])
def test_forward_matches_oracle(case, T):
    cfg, layer, ref = case
    log(f"{cfg.name} forward T={T}")
    x = synth.tokens(cfg, T=T, stream=T)
    xd = torch.from_numpy(x).cuda()
    out = layer.forward(xd, 0).cpu().numpy()
    ids, w = layer.route(xd, 0)
    rc, missing = layer.status()
    assert rc == 0, missing
    r_out, r_ids, r_w, gk, gi = ref.forward(x)
    check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, f"{cfg.name} T={T}")
    excluded, _ = flags(gk, gi)
    err = rel_err(out, r_out, ~excluded)
    log(f"  max|d|/max|ref| = {err:.3e}, flagged {int(excluded.sum())}/{T}")
    assert err <= REL_TOL


def test_groups_change_the_selection(case):
    """The group step is active: for some tokens the group-limited choice
    differs from plain top-K on the same scores."""
    cfg, layer, ref = case
    x = synth.tokens(cfg, T=64, stream=7)
    ids_g, *_ = oracle.route(x, ref.W, ref.b, cfg.K, cfg.routed_scale, cfg.norm_topk,
                             cfg.n_group, cfg.topk_group)
    ids_p, *_ = oracle.route(x, ref.W, ref.b, cfg.K, cfg.routed_scale, cfg.norm_topk)
    differ = sum(set(a.tolist()) != set(b.tolist()) for a, b in zip(ids_g, ids_p))
    log(f"{cfg.name}: {differ}/64 tokens choose differently with groups")
    assert differ > 0
    ids, _ = layer.route(torch.from_numpy(x).cuda(), 0)
    ids = ids.cpu().numpy()
    gsz = cfg.E // cfg.n_group
    for t in range(64):
        assert len(set((ids[t] // gsz).tolist())) <= cfg.topk_group
