"""Parity of the many-token router (more than 16 tokens), which forms the
logits on the fp16 matrix cores from hi/lo fp16 halves of the fp32 operands
after exact power-of-two scales (per token from its sum of squares, per
expert from its largest weight): ids exact against the oracle outside near
ties, weights to 1e-5, as every routing test.

- Every expert count the kernel is specialised on (2, 4, 6 and 8
  wavefronts of 32 experts: E = 32, 96, 160, 256), at token counts that
  fill one, two and three 128-token workgroups with a ragged tail.
- Inputs scaled by 1e-6 and 1e2 through the residual form, whose routing
  sees rmsnorm(x): the router's token scale must absorb the factor
  (unscaled fp16 halves would lose 1e-6-sized values to subnormals; at 1e2
  the routing is the unscaled one, at 1e-6 the RMSNorm epsilon shrinks the
  logits on both sides alike).  The new x and the MoE term alone are
  checked (max|d|/max|ref| <= 2e-3).
- Weights whose rows differ by powers of ten in magnitude (the per-expert
  scale)."""
import numpy as np
import pytest

import synth
from synth.configs import LayerConfig, W_INT4_ROW
from parity import OracleLayer, check_ids, check_residual, flags, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import workload  # noqa: E402


def cfg(name, E, K, seed, H=512, I=256):
    return LayerConfig(name, H=H, I=I, E=E, K=K, n_shared=1, fmt=W_INT4_ROW, T=1, n_layers=1,
                       seed=seed, zipf_c=0.2)


@pytest.mark.parametrize("E,K", [(32, 4), (96, 8), (160, 8), (256, 8)])
def test_route_every_wavefront_count(E, K):
    c = cfg(f"router_e{E}", E, K, seed=940 + E)
    Ts = (17, 130, 300)
    log(f"case {c.name}: H={c.H} E={E} K={K} T={Ts}")
    ml = workload.build_layer(c, max_tokens=max(Ts))
    ref = OracleLayer(c, 0)
    try:
        for T in Ts:
            x = synth.tokens(c, T=T, stream=T)
            ids, w = ml.route(torch.from_numpy(x).cuda(), 0)
            assert ml.status()[0] == 0
            r_ids, r_w, _, _, gk, gi = ref.route(x)
            n_ex = check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi,
                             f"{c.name} T={T}")
            log(f"{c.name} T={T}: ids exact (flagged {n_ex})")
    finally:
        ml.close()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("scale", [1e-6, 1e2])
def test_residual_scale_free_routing(scale):
    c = cfg("router_scaled", 64, 8, seed=951)
    T = 200
    log(f"case {c.name}: E={c.E} K={c.K} T={T} x scaled by {scale:g}")
    ml = workload.build_layer(c, max_tokens=T)
    ref = OracleLayer(c, 0)
    try:
        x = (synth.tokens(c, T=T, stream=7).astype(np.float64) * scale).astype(np.float32)
        xd = torch.from_numpy(x.copy()).cuda()
        got = ml.forward_residual(xd, 0).cpu().numpy()
        assert ml.status()[0] == 0
        r_next, r_ids, r_w, gk, gi = ref.forward(x, residual=True)
        excluded, _ = flags(gk, gi)
        e_next, e_term = check_residual(x, got, r_next, ~excluded, f"scale {scale:g}")
        log(f"scale {scale:g}: new x {e_next:.2e}, moe term {e_term:.2e} "
            f"(flagged {int(excluded.sum())})")
    finally:
        ml.close()
        torch.cuda.empty_cache()


def test_route_rows_of_different_magnitude():
    """Router rows scaled by 10^(e mod 7 - 3): each expert's own power of two
    must keep its logits at fp32 accuracy (a shared scale would push the
    small rows' low halves into fp16 subnormals)."""
    c = cfg("router_rows", 64, 4, seed=952)
    T = 150
    ml = workload.build_layer(c, max_tokens=T)
    ref = OracleLayer(c, 0)
    try:
        f = (10.0 ** (np.arange(c.E) % 7 - 3)).astype(np.float32)
        W = (ref.W.astype(np.float64) * f[:, None]).astype(np.float32)
        ref.W = W
        ml.set_router(0, W, ref.b)
        x = synth.tokens(c, T=T, stream=11)
        ids, w = ml.route(torch.from_numpy(x).cuda(), 0)
        assert ml.status()[0] == 0
        r_ids, r_w, _, _, gk, gi = ref.route(x)
        n_ex = check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, c.name)
        log(f"{c.name} T={T}: ids exact (flagged {n_ex})")
    finally:
        ml.close()
        torch.cuda.empty_cache()
