"""The few-token matrix-core path (row format, 9 .. 63 tokens: the row
router up to 16 tokens, the k-sliced gate/up and down units on
v_mfma_f32_16x16x32_f16, the h rows kernel, the combine) against the oracle
through the C ABI.  Shapes chosen for its variants: one and several k-slices,
a shared expert with more than 16 tokens (several passes over the codes),
K up to 8, the residual form, a missing expert and bitwise determinism; the
GLM shape at 33 tokens (a verify-sized batch past the GEMVs' range)."""
import numpy as np
import pytest

import synth
from parity import OracleLayer, WORKERS, check_ids, check_residual, flags, log, rel_err, REL_TOL
from synth.configs import LayerConfig, W_INT4_ROW

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M, workload  # noqa: E402

CASES = {
    # name: (H, I, E, K, n_shared)
    "h1024": (1024, 512, 32, 4, 1),
    "h2048": (2048, 1024, 64, 8, 1),
    "h3072": (3072, 768, 48, 6, 0),
}
TS = [9, 16, 17, 33, 63]


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    H, I, E, K, ns = CASES[request.param]
    cfg = LayerConfig(name=f"midt_{request.param}", H=H, I=I, E=E, K=K, n_shared=ns, fmt=W_INT4_ROW,
                      T=63, n_layers=1, seed=990 + list(CASES).index(request.param), zipf_c=0.2)
    ml = workload.build_layer(cfg, max_tokens=63)
    yield cfg, ml, OracleLayer(cfg, 0)
    ml.close()


@pytest.mark.parametrize("T", TS)
def test_forward(case, T):
    cfg, ml, ref = case
    x = synth.tokens(cfg, T=T, stream=T)
    xd = torch.from_numpy(x).cuda()
    out = ml.forward(xd, 0).cpu().numpy()
    ids, w = ml.route(xd, 0)
    assert ml.status()[0] == M.MOE_OK
    r_out, r_ids, r_w, gk, gi = ref.forward(x, workers=WORKERS)
    check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, f"{cfg.name} T={T}")
    excluded, _ = flags(gk, gi)
    err = rel_err(out, r_out, ~excluded)
    log(f"{cfg.name} T={T}: max|d|/max|ref| = {err:.2e}, flagged {int(excluded.sum())}")
    assert err <= REL_TOL


@pytest.mark.parametrize("T", [9, 33])
def test_residual(case, T):
    cfg, ml, ref = case
    x = synth.tokens(cfg, T=T, stream=40 + T)
    xd = torch.from_numpy(x).cuda()
    ml.forward_residual(xd, 0)
    got = xd.cpu().numpy()
    r_next, _, _, gk, gi = ref.forward(x, residual=True, workers=WORKERS)
    excluded, _ = flags(gk, gi)
    e_next, e_term = check_residual(x, got, r_next, ~excluded, f"{cfg.name} T={T} residual")
    log(f"{cfg.name} T={T} residual: {e_next:.2e} (new x), {e_term:.2e} (moe term)")
    assert ml.status()[0] == M.MOE_OK


def test_deterministic_and_missing_expert(case):
    cfg, ml, ref = case
    T = 17
    x = synth.tokens(cfg, T=T, stream=77)
    xd = torch.from_numpy(x).cuda()
    a = ml.forward(xd, 0).clone()
    b = ml.forward(xd, 0).clone()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    r_out, r_ids, r_w, gk, gi = ref.forward(x, workers=WORKERS)
    victim = int(r_ids[0, 0])
    ml.map(0, victim, -1)
    try:
        out = ml.forward(xd, 0).cpu().numpy()
        rc, missing = ml.status()
        assert rc == M.MOE_E_NOT_RESIDENT and missing == [victim]
        # the reference without the victim: its weighted output removed from
        # every token that chose it
        y = {}
        want = r_out.astype(np.float64).copy()
        for t in range(T):
            for k in range(cfg.K):
                if int(r_ids[t, k]) == victim:
                    if t not in y:
                        y[t], _ = __import__("oracle").expert(cfg.fmt, cfg.H, cfg.I, ref.cache[victim], x[t])
                    want[t] -= float(r_w[t, k]) * y[t].astype(np.float64)
        excluded, _ = flags(gk, gi)
        err = rel_err(out, want, ~excluded)
        log(f"{cfg.name} without expert {victim}: max|d|/max|ref| = {err:.2e}")
        assert err <= REL_TOL
    finally:
        ml.map(0, victim, victim)


def test_glm_33_tokens():
    """The GLM shape at 33 tokens: every token's routing, the outputs of 8
    tokens spread over the batch."""
    cfg = synth.CONFIGS["glm_verify"]
    ml = workload.build_layer(cfg, n_layers=1, max_tokens=33)
    try:
        ref = OracleLayer(cfg, 0)
        T = 33
        x = synth.tokens(cfg, T=T, stream=9)
        xd = torch.from_numpy(x).cuda()
        out = ml.forward(xd, 0).cpu().numpy()
        ids, w = ml.route(xd, 0)
        assert ml.status()[0] == M.MOE_OK
        r_ids, r_w, _, _, gk, gi = ref.route(x)
        check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, "glm T=33")
        excluded, _ = flags(gk, gi)
        pick = [t for t in range(0, T, 4) if not excluded[t]][:8]
        r_out, _, _, _, _ = ref.forward(x[pick], workers=WORKERS)
        err = rel_err(out[pick], r_out)
        log(f"glm T=33: outputs of tokens {pick}: max|d|/max|ref| = {err:.2e}")
        assert err <= REL_TOL
    finally:
        ml.close()
        torch.cuda.empty_cache()
