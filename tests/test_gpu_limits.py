"""Parity at the limits the library accepts and in the method's degenerate
cases: the largest hidden size (16384), the grouped GEMM's largest
intermediate size (8192), 256 experts with top-8, every expert chosen
(K = E), top-1, an all-zero input, and the bucketing maximum of 65536
assignments.  Same rules as the other parity tests (ids exact outside near
ties, max|d|/max|ref| <= 2e-3)."""
import os

import numpy as np
import pytest

import synth
from synth.configs import LayerConfig, W_INT4_AFFINE_G64, W_INT4_ROW
from parity import OracleLayer, check_ids, flags, log, rel_err, REL_TOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import workload  # noqa: E402


def cfg(name, H, I, E, K, n_shared=1, fmt=W_INT4_ROW, seed=900, **kw):
    return LayerConfig(name, H=H, I=I, E=E, K=K, n_shared=n_shared, fmt=fmt, T=1, n_layers=1,
                       seed=seed, zipf_c=0.2, **kw)


CASES = {
    "max_hidden_row": (cfg("max_hidden_row", 16384, 256, 16, 2, seed=901), (1, 5, 40)),
    "max_hidden_affine": (cfg("max_hidden_affine", 16384, 512, 16, 2, 0, W_INT4_AFFINE_G64,
                              seed=902), (1, 9)),
    "max_inter_gemm": (cfg("max_inter_gemm", 512, 8192, 8, 2, seed=903), (1, 64, 130)),
    "e256_top8": (cfg("e256_top8", 256, 256, 256, 8, seed=904), (1, 8, 33)),
    "every_expert": (cfg("every_expert", 512, 256, 8, 8, seed=905), (1, 3, 70)),
    "top1": (cfg("top1", 512, 256, 16, 1, seed=906), (1, 8, 100)),
    # the small router's largest partial region at several tokens: 64 column
    # slices x 8 tokens x 4 expert blocks, each block summed by its own last
    # workgroup
    "max_hidden_e256": (cfg("max_hidden_e256", 16384, 256, 256, 2, seed=909), (8, 3)),
}


def run_case(c, Ts, zero=False):
    log(f"case {c.name}: H={c.H} I={c.I} E={c.E} K={c.K} fmt={c.fmt} T={Ts}")
    ml = workload.build_layer(c, max_tokens=max(Ts))
    ref = OracleLayer(c, 0)
    try:
        for T in Ts:
            x = synth.tokens(c, T=T, stream=T)
            if zero:
                x = np.zeros_like(x)
            xd = torch.from_numpy(x).cuda()
            out = ml.forward(xd, 0).cpu().numpy()
            ids, w = ml.route(xd, 0)
            assert ml.status()[0] == 0
            r_out, r_ids, r_w, gk, gi = ref.forward(x)
            check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, f"{c.name} T={T}")
            excluded, _ = flags(gk, gi)
            keep = np.ones(T, bool) if zero else ~excluded
            err = rel_err(out, r_out, keep) if np.abs(r_out).max() > 0 else float(np.abs(out).max())
            log(f"{c.name} T={T}: max|d|/max|ref| = {err:.2e} (flagged {int(excluded.sum())})")
            assert err <= REL_TOL
    finally:
        ml.close()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", list(CASES))
def test_limits(name):
    c, Ts = CASES[name]
    run_case(c, Ts)


def test_zero_input():
    """x = 0: every logit is 0 and sigma(0) = 0.5 exactly on both sides, so the
    choice falls to the bias (ids must match); every output is 0."""
    c = cfg("zero_input", 512, 256, 32, 4, seed=907)
    run_case(c, (1, 6, 64), zero=True)


def test_bucketing_maximum():
    """T*K = 65536 assignments (8192 tokens, top-8) on a small layer, through
    the large-T router and the grouped GEMM; outputs of every token."""
    c = cfg("bucket_max", 512, 256, 64, 8, seed=908)
    T = 8192
    log("case bucket_max: H=512 I=256 E=64 K=8 T=8192")
    ml = workload.build_layer(c, max_tokens=T)
    ref = OracleLayer(c, 0)
    try:
        x = synth.tokens(c, T=T, stream=3)
        xd = torch.from_numpy(x).cuda()
        out = ml.forward(xd, 0).cpu().numpy()
        ids, w = ml.route(xd, 0)
        assert ml.status()[0] == 0
        r_out, r_ids, r_w, gk, gi = ref.forward(x, workers=min(16, os.cpu_count() or 1))
        check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, "bucket_max")
        excluded, _ = flags(gk, gi)
        err = rel_err(out, r_out, ~excluded)
        log(f"bucket_max T={T}: all tokens max|d|/max|ref| = {err:.2e}")
        assert err <= REL_TOL
    finally:
        ml.close()
        torch.cuda.empty_cache()
