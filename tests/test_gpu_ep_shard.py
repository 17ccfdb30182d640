"""One GPU's share of an expert-parallel layer: the experts held elsewhere
are marked MOE_SLOT_REMOTE in the slot table.  A forward then raises no
status and returns the partial sum this GPU owes: the shared expert plus
the weighted outputs of the local routed experts, the routing (ids and
weights, renormalised over all K) unchanged.  Checked against the oracle
with the remote experts' weighted outputs removed, on the one-token path
(the gate/up kernel's selection) and on several tokens (the router tail and
the top-K kernel)."""
import numpy as np
import pytest

import oracle
import synth
from parity import OracleLayer, WORKERS, flags, log, rel_err, REL_TOL
from synth.configs import LayerConfig, W_INT4_ROW

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M, workload  # noqa: E402

# tiny: general paths; h2048: the one-token kernels with the selection in the
# gate/up kernel (H a multiple of 2048, sigmoid, one group)
CASES = {
    "tiny": synth.CONFIGS["tiny"],
    "h2048": LayerConfig(name="ep_h2048", H=2048, I=512, E=64, K=8, n_shared=1, fmt=W_INT4_ROW,
                         T=1, n_layers=1, seed=995, zipf_c=0.2),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    cfg = CASES[request.param]
    ml = workload.build_layer(cfg, max_tokens=64)
    yield cfg, ml, OracleLayer(cfg, 0)
    ml.close()


@pytest.mark.parametrize("T", [1, 5, 40])
def test_remote_experts_give_the_local_partial_sum(case, T):
    cfg, ml, ref = case
    remote = [e for e in range(cfg.E) if e % 2 == 1]
    x = synth.tokens(cfg, T=T, stream=60 + T)
    for e in remote:
        ml.map(0, e, M.MOE_SLOT_REMOTE)
    try:
        out = ml.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
        rc, missing = ml.status()
        assert rc == M.MOE_OK and missing == [], (rc, missing)
    finally:
        for e in remote:
            ml.map(0, e, e)
    r_out, r_ids, r_w, gk, gi = ref.forward(x, workers=WORKERS)
    want = r_out.astype(np.float64).copy()
    for t in range(T):
        for k in range(cfg.K):
            e = int(r_ids[t, k])
            if e % 2 == 1:
                y, _ = oracle.expert(cfg.fmt, cfg.H, cfg.I, ref.cache[e], x[t])
                want[t] -= float(r_w[t, k]) * y.astype(np.float64)
    excluded, _ = flags(gk, gi)
    err = rel_err(out, want, ~excluded)
    n_remote = int(np.sum(r_ids % 2 == 1))
    log(f"{cfg.name} T={T}: {n_remote} of {T * cfg.K} assignments remote; local partial sum "
        f"max|d|/max|ref| = {err:.2e}")
    assert err <= REL_TOL


def test_remote_slot_value_is_checked(case):
    cfg, ml, _ = case
    assert M.moe_map_expert(ml.ctx, 0, 0, -3) == M.MOE_E_SLOT
    assert M.moe_map_expert(ml.ctx, 0, 0, M.MOE_SLOT_REMOTE) == M.MOE_OK
    assert M.moe_map_expert(ml.ctx, 0, 0, 0) == M.MOE_OK
