"""Full-size parity on the Edge0 shape (H=2048, E=256, I=512, no shared
expert, affine int4 with group size 64) through the C ABI: a 40-layer decode
step chained by x <- x + moe(rmsnorm(x)), top-4 and top-8, every layer
teacher-forced against the oracle, plus the free-running chain reported."""
import numpy as np
import pytest

import synth
from parity import OracleLayer, flags, log, rel_err, REL_TOL, check_residual

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import workload  # noqa: E402


@pytest.mark.parametrize("name", ["edge0_decode", "edge0_decode_k8"])
def test_edge0_40_layers(name):
    cfg = synth.CONFIGS[name]
    log(f"building {name}: 40 layers x 256 affine experts")
    ml = workload.build_layer(cfg)
    try:
        x = synth.tokens(cfg, T=1)
        xg = torch.from_numpy(x).cuda()
        worst, worst_term, n_flag = 0.0, 0.0, 0
        for layer in range(cfg.n_layers):
            ref = OracleLayer(cfg, layer)
            r_next, r_ids, r_w, gk, gi = ref.forward(x, residual=True)
            xt = torch.from_numpy(x).cuda()
            ml.forward_residual(xt, layer)
            ml.forward_residual(xg, layer)
            excluded, _ = flags(gk, gi)
            if excluded[0]:
                n_flag += 1
            else:
                e_next, e_term = check_residual(x, xt.cpu().numpy(), r_next, None,
                                                f"{name} layer {layer}")
                worst = max(worst, e_next)
                worst_term = max(worst_term, e_term)
            x = r_next
        chain = rel_err(xg.cpu().numpy(), x)
        log(f"{name}: worst per-layer max|d|/max|ref| = {worst:.3e} (new x), {worst_term:.3e} "
            f"(moe term), flagged layers {n_flag}, "
            f"end-to-end chained (reported) {chain:.3e}")
        rc, _ = ml.status()
        assert rc == 0
    finally:
        ml.close()
        torch.cuda.empty_cache()
