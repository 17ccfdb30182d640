"""The one-token kernels (gate/up straight to h, down with the combine, each
workgroup reducing 8 whole rows) against the oracle through the C ABI, on
shapes chosen to exercise their launch variants: 1, 2, 3 and 4 wavefronts
per gate/up workgroup and 1 to 4 steps per wavefront, both weight formats,
with and without a shared expert, K up to 8 (nine expert slots in the down
workgroup), the residual form, a missing expert and bitwise determinism.
The GLM and Edge0 decode tests run these kernels at full size."""
import numpy as np
import pytest

import synth
from parity import OracleLayer, check_ids, check_residual, flags, log, rel_err, REL_TOL
from synth.configs import LayerConfig, W_INT4_AFFINE_G64, W_INT4_ROW

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M, workload  # noqa: E402

CASES = {
    # name: (H, I, E, K, n_shared, fmt)  -- gate/up waves x steps, down steps
    "r512": (512, 512, 32, 4, 1, W_INT4_ROW),            # 1 wave x 1 step, down 1 step
    "r1024": (1024, 1024, 64, 8, 1, W_INT4_ROW),         # 2 x 1, down 2, nine slots
    "a1536": (1536, 512, 32, 4, 0, W_INT4_AFFINE_G64),   # 3 x 1, no shared expert
    "r4096": (4096, 1536, 64, 8, 1, W_INT4_ROW),         # 4 x 2, down 3
    "a6144": (6144, 2048, 32, 6, 1, W_INT4_AFFINE_G64),  # 4 x 3, down 4
    "r8192": (8192, 512, 32, 2, 1, W_INT4_ROW),          # 4 x 4, down 1
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    H, I, E, K, ns, fmt = CASES[request.param]
    cfg = LayerConfig(name=f"tok1_{request.param}", H=H, I=I, E=E, K=K, n_shared=ns, fmt=fmt,
                      T=1, n_layers=1, seed=970 + list(CASES).index(request.param), zipf_c=0.2)
    ml = workload.build_layer(cfg, max_tokens=4)
    yield cfg, ml, OracleLayer(cfg, 0)
    ml.close()


def test_forward_and_residual(case):
    cfg, ml, ref = case
    for s in range(3):
        x = synth.tokens(cfg, T=1, stream=s)
        xd = torch.from_numpy(x).cuda()
        out = ml.forward(xd, 0).cpu().numpy()
        ids, w = ml.route(xd, 0)
        r_out, r_ids, r_w, gk, gi = ref.forward(x)
        check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, cfg.name)
        excluded, _ = flags(gk, gi)
        err = rel_err(out, r_out, ~excluded)
        log(f"{cfg.name} stream {s}: max|d|/max|ref| = {err:.2e}")
        assert err <= REL_TOL
    x = synth.tokens(cfg, T=1, stream=9) * 2.0
    xd = torch.from_numpy(x).cuda()
    ml.forward_residual(xd, 0)
    r_next, _, _, gk, gi = ref.forward(x, residual=True)
    excluded, _ = flags(gk, gi)
    e_next, e_term = check_residual(x, xd.cpu().numpy(), r_next, ~excluded, cfg.name)
    log(f"{cfg.name} residual: {e_next:.2e} (new x), {e_term:.2e} (moe term)")
    assert ml.status()[0] == M.MOE_OK


def test_deterministic_and_missing_expert(case):
    cfg, ml, ref = case
    x = synth.tokens(cfg, T=1, stream=20)
    xd = torch.from_numpy(x).cuda()
    a = ml.forward(xd, 0).clone()
    b = ml.forward(xd, 0).clone()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    _, r_ids, r_w, gk, gi = ref.forward(x)
    victim = int(r_ids[0, cfg.K - 1])
    ml.map(0, victim, -1)
    try:
        out = ml.forward(xd, 0).cpu().numpy()
        rc, missing = ml.status()
        assert rc == M.MOE_E_NOT_RESIDENT and missing == [victim]
        # the reference without the victim: its weight times its output removed
        blobs = ref.cache
        y_v, _ = __import__("oracle").expert(cfg.fmt, cfg.H, cfg.I, blobs[victim], x[0])
        want = ref.forward(x)[0][0] - float(r_w[0, cfg.K - 1]) * y_v.astype(np.float64)
        err = rel_err(out[0], want)
        log(f"{cfg.name} without expert {victim}: max|d|/max|ref| = {err:.2e}")
        assert err <= REL_TOL
    finally:
        ml.map(0, victim, victim)


def test_non_finite_input_is_reported(case):
    """A NaN or an infinity in the token sets MOE_E_RANGE on the one-token
    router too (its first workgroup forms the token's sum of squares); the
    status clears, and the next finite forward is clean and matches."""
    cfg, ml, ref = case
    x = synth.tokens(cfg, T=1, stream=30)
    for bad in (np.nan, np.inf):
        xb = x.copy()
        xb[0, cfg.H // 3] = bad
        ml.forward(torch.from_numpy(xb).cuda(), 0)
        rc, missing = ml.status()
        assert rc == M.MOE_E_RANGE and missing == [], (bad, rc)
        assert ml.status()[0] == M.MOE_OK
    out = ml.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
    assert ml.status()[0] == M.MOE_OK
    r_out, _, _, gk, gi = ref.forward(x)
    excluded, _ = flags(gk, gi)
    err = rel_err(out, r_out, ~excluded)
    log(f"{cfg.name} after the non-finite inputs: max|d|/max|ref| = {err:.2e}")
    assert err <= REL_TOL
