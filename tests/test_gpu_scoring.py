"""Parity of softmax scoring through the C ABI: renormalised weights (row
format with a shared expert) and raw probabilities (affine), over the small-T
router tail (T <= 8), the large-T top-k with the GEMV path (T = 20) and with
the grouped GEMM (T = 64, row format)."""
import numpy as np
import pytest

import oracle
import synth
from parity import OracleLayer, check_ids, flags, log, rel_err, REL_TOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import workload  # noqa: E402

TMAX = 64


@pytest.fixture(scope="module", params=["softmax_renorm", "softmax_raw"])
def case(request):
    cfg = synth.CONFIGS[request.param]
    ml = workload.build_layer(cfg, max_tokens=TMAX)
    yield cfg, ml, OracleLayer(cfg, 0)
    ml.close()


@pytest.mark.parametrize("T", [1, 4, 8, 20, TMAX])
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


def test_weights_follow_the_scoring(case):
    """Renormalised: the weights of a token sum to routed_scale; raw: they are
    the chosen softmax probabilities, summing to less than routed_scale."""
    cfg, layer, ref = case
    x = synth.tokens(cfg, T=16, stream=5)
    _, w = layer.route(torch.from_numpy(x).cuda(), 0)
    s = w.cpu().numpy().astype(np.float64).sum(axis=1)
    if cfg.norm_topk:
        assert np.allclose(s, cfg.routed_scale, atol=1e-5)
    else:
        assert np.all(s < cfg.routed_scale) and np.all(s > 0)
