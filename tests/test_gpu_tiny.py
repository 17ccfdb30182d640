"""Parity of the whole layer on the tiny shape (H=512, E=32, top-4, I=256, one
shared expert) through the C ABI: all token counts of the decode path, the
prefill path, the residual form, missing experts, determinism."""
import numpy as np
import pytest

import oracle
import synth
from parity import OracleLayer, check_ids, flags, log, rel_err, REL_TOL, check_residual

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M  # noqa: E402
from int4_weight_expert_amd import workload  # noqa: E402

CFG = synth.CONFIGS["tiny"]
TMAX = 300


@pytest.fixture(scope="module")
def layer():
    ml = workload.build_layer(CFG, max_tokens=TMAX)
    yield ml
    ml.close()


@pytest.fixture(scope="module")
def ref():
    return OracleLayer(CFG, 0)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 8, 9, 16, 17, 64, 129, TMAX])
def test_forward_matches_oracle(layer, ref, T):
    log(f"tiny forward T={T}")
    x = synth.tokens(CFG, T=T, stream=T)
    out = layer.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
    ids, w = layer.route(torch.from_numpy(x).cuda(), 0)
    rc, missing = layer.status()
    assert rc == 0, missing
    r_out, r_ids, r_w, gk, gi = ref.forward(x)
    check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, f"T={T}")
    excluded, _ = flags(gk, gi)
    err = rel_err(out, r_out, ~excluded)
    log(f"  max|d|/max|ref| = {err:.3e}, flagged {int(excluded.sum())}/{T}")
    assert err <= REL_TOL


@pytest.mark.parametrize("T", [1, 4, 16, 33])
def test_residual_matches_oracle(layer, ref, T):
    log(f"tiny residual T={T}")
    x = synth.tokens(CFG, T=T, stream=100 + T) * 3.0
    xd = torch.from_numpy(x).cuda()
    layer.forward_residual(xd, 0)
    r_out, r_ids, r_w, gk, gi = ref.forward(x, residual=True)
    excluded, _ = flags(gk, gi)
    e_next, e_term = check_residual(x, xd.cpu().numpy(), r_out, ~excluded, f"T={T}")
    log(f"  max|d|/max|ref| = {e_next:.3e} (new x), {e_term:.3e} (moe term)")


def test_deterministic(layer):
    for T in (1, 8, 200):
        x = torch.from_numpy(synth.tokens(CFG, T=T, stream=7)).cuda()
        a = layer.forward(x, 0).clone()
        b = layer.forward(x, 0).clone()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), T


def test_missing_expert_is_reported_and_skipped(layer, ref):
    T = 4
    x = synth.tokens(CFG, T=T, stream=11)
    _, r_ids, r_w, gk, gi = ref.forward(x)
    victim = int(r_ids[0, 0])
    layer.map(0, victim, -1)
    try:
        out = layer.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
        rc, missing = layer.status()
        assert rc == M.MOE_E_NOT_RESIDENT
        assert missing == [victim]
        rc2, _ = layer.status()
        assert rc2 == 0                       # cleared
        # expected: the victim contributes zero
        blobs = [None if e == victim else ref.cache.get(e) for e in range(CFG.E)]
        ref.need(r_ids)
        blobs = [None if e == victim else ref.cache.get(e) for e in range(CFG.E)]
        for t in range(T):
            acc = np.zeros(CFG.H)
            for s in range(CFG.n_shared):
                acc += oracle.expert(CFG.fmt, CFG.H, CFG.I, ref.shared[s], x[t])[0]
            for k in range(CFG.K):
                e = int(r_ids[t, k])
                if blobs[e] is not None:
                    acc += float(r_w[t, k]) * oracle.expert(CFG.fmt, CFG.H, CFG.I, blobs[e], x[t])[0]
            assert rel_err(out[t], acc) <= REL_TOL
    finally:
        layer.map(0, victim, victim)


def test_load_expert_blob_path(layer, ref):
    """Experts loaded from oracle-packed blobs give the same forward."""
    T = 5
    x = synth.tokens(CFG, T=T, stream=21)
    ml = workload.MoeLayer(CFG.H, CFG.I, CFG.E, CFG.K, CFG.n_shared, 1, CFG.fmt, n_slots=CFG.E,
                           max_tokens=T)
    try:
        W, b = synth.router_weight(CFG, 0), synth.router_bias(CFG, 0)
        ml.set_router(0, W, b)
        ref.need(range(CFG.E))
        for e in range(CFG.E):
            ml.load_expert(e, ref.cache[e])
            ml.map(0, e, e)
        ml.set_shared(0, 0, ref.shared[0])
        a = ml.forward(torch.from_numpy(x).cuda(), 0)
        b2 = layer.forward(torch.from_numpy(x).cuda(), 0)
        assert torch.equal(a, b2)
    finally:
        ml.close()


def test_graph_replay_matches_eager(layer):
    """Forwards captured in a HIP graph: every replay, with eager work and
    synchronisation between replays, equals the eager result."""
    # T = 1 and 8: the GEMV path (8: the router's per-block reductions);
    # T = 4: gate/up as one workgroup per (group, block); T = 64: the
    # grouped-GEMM path
    xs = [torch.from_numpy(synth.tokens(CFG, T=T, stream=30 + T)).cuda() for T in (1, 4, 8, 64)]
    eager = [layer.forward(x, 0).clone() for x in xs]
    outs = [torch.empty_like(x) for x in xs]
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    M.moe_set_stream(layer.ctx, cap.cuda_stream)
    try:
        with torch.cuda.graph(g, stream=cap):
            for x, o in zip(xs, outs):
                M._check("moe_forward", M.moe_forward(layer.ctx, x, x.shape[0], 0, o))
    finally:
        M.moe_set_stream(layer.ctx, torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), rep
        other = layer.forward(torch.from_numpy(synth.tokens(CFG, T=3, stream=99)).cuda(), 0)
        torch.cuda.synchronize()
        assert torch.isfinite(other).all()
