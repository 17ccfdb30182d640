"""Per-row int8 shared experts ([GLM-C] §05 quantize_rows, bits = 8): the
device quantiser bit-exact against the oracle, the shared slot's bytes, and
layer forwards (T = 1 .. 64, plain and residual) against the oracle with
the routed experts in int4 and the shared expert in int8."""
import numpy as np
import pytest

import oracle
import synth
from parity import (OracleLayer, WORKERS, block_sample, check_ids, check_residual, flags, log,
                    oracle_blob, rel_err, REL_TOL)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M, workload  # noqa: E402
from int4_weight_expert_amd.layer import MoeLayer  # noqa: E402

KINDS = {"f32": oracle.SRC_F32, "bf16": oracle.SRC_BF16, "fp8": oracle.SRC_FP8_E4M3}


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("O,I", [(130, 256), (64, 2048), (7, 6)])
def test_int8_quantiser_bit_exact(kind, O, I):
    k = synth.key(950, 0, O, I)
    if kind == "fp8":
        w, sinv = synth.fp8_checkpoint(k, O, I, 0.02)
    elif kind == "bf16":
        w, sinv = synth.bf16_checkpoint(k, O, I, 0.02), None
    else:
        w, sinv = synth.gauss(k, O * I, 0.02).reshape(O, I), None
    w = w.copy()
    if O > 2:
        w[0] = 0
    src = torch.from_numpy(w.view(np.int16) if w.dtype == np.uint16 else w).cuda()
    si = None if sinv is None else torch.from_numpy(sinv).cuda()
    q = torch.empty((O, I), dtype=torch.int8, device="cuda")
    s = torch.empty(O, dtype=torch.float32, device="cuda")
    M._check("moe_requant_int8_rows", M.moe_requant_int8_rows(src, KINDS[kind], si, O, I, q, s, 0))
    torch.cuda.synchronize()
    rq, rs = oracle.pack_int8_row(oracle.decode_source(w, KINDS[kind], sinv))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.fixture(scope="module", params=["int8_shared", "mid_int8_shared", "affine_int8_shared"])
def case(request):
    cfg = synth.CONFIGS[request.param]
    ml = workload.build_layer(cfg, max_tokens=64)
    yield cfg, ml, OracleLayer(cfg, 0)
    ml.close()


def test_shared_slot_bytes(case):
    cfg, ml, _ = case
    assert ml.shared_bytes == oracle.blob_bytes(oracle.W_INT8_ROW, cfg.H, cfg.I)
    assert np.array_equal(ml.read_shared(0, 0), oracle_blob(cfg, 0, cfg.E))


@pytest.mark.parametrize("T", [1, 3, 8, 20, 64])
@pytest.mark.parametrize("residual", [False, True])
def test_forward_matches_oracle(case, T, residual):
    cfg, ml, ref = case
    x = synth.tokens(cfg, T=T, stream=T)
    xd = torch.from_numpy(x).cuda()
    if residual:
        got = ml.forward_residual(xd.clone(), 0).cpu().numpy()
    else:
        got = ml.forward(xd, 0).cpu().numpy()
        ids, w = ml.route(xd, 0)
    assert ml.status()[0] == 0
    r_out, r_ids, r_w, gk, gi = ref.forward(x, residual=residual)
    if not residual:
        check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, f"{cfg.name} T={T}")
    excluded, _ = flags(gk, gi)
    if residual:
        err, term = check_residual(x, got, r_out, ~excluded, f"{cfg.name} T={T}")
        log(f"{cfg.name} T={T} residual: max|d|/max|ref| = {err:.2e} (new x), {term:.2e} "
            f"(moe term)")
    else:
        err = rel_err(got, r_out, ~excluded)
        log(f"{cfg.name} T={T}: max|d|/max|ref| = {err:.2e}")
        assert err <= REL_TOL


def test_blob_path_and_errors():
    cfg = synth.CONFIGS["int8_shared"]
    ml = MoeLayer(cfg.H, cfg.I, cfg.E, cfg.K, 1, 1, cfg.fmt, n_slots=1, max_tokens=4,
                  shared_fmt=oracle.W_INT8_ROW)
    try:
        blob = oracle_blob(cfg, 0, cfg.E)
        ml.set_shared(0, 0, blob)
        assert np.array_equal(ml.read_shared(0, 0), blob)
        assert M.moe_set_shared(ml.ctx, 0, 0, blob, blob.nbytes - 1) == M.MOE_E_SIZE
        q = np.zeros(cfg.I * cfg.H // 2, np.uint8)
        s = np.zeros(cfg.H, np.float32)
        assert M.moe_import_shared(ml.ctx, 0, 0, q, q, q, s, s, s) == M.MOE_E_UNSUPPORTED
    finally:
        ml.close()
    bad = M.make_config(cfg.H, cfg.I, cfg.E, cfg.K, 1, 1, cfg.fmt, 1, 4, shared_fmt=2)
    assert M.moe_layer_create_rc(bad)[0] == M.MOE_E_ARG


def test_glm_decode_int8_shared():
    cfg = synth.CONFIGS["glm_decode_int8_shared"]
    ml = workload.build_layer(cfg, n_layers=1, max_tokens=2)
    ref = OracleLayer(cfg, 0)
    try:
        for T in (1, 2):
            x = synth.tokens(cfg, T=T, stream=T)
            got = ml.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
            r_out, _, _, gk, gi = ref.forward(x)
            excluded, _ = flags(gk, gi)
            err = rel_err(got, r_out, ~excluded)
            log(f"GLM decode, int8 shared, T={T}: max|d|/max|ref| = {err:.2e}")
            assert err <= REL_TOL
    finally:
        ml.close()


@pytest.mark.parametrize("name", ["int8_shared", "affine_int8_shared"])
def test_int8_shared_several_layers(name):
    """Three layers with int8 shared experts: each layer's shared slot (its
    own stride, not the routed slot size) reads back as the oracle's blob
    after the device pack, after a host blob (the last layer) and after a
    requantised fp32 source (layer 1), and a forward on every layer matches
    the oracle."""
    cfg = synth.CONFIGS[name].with_(n_layers=3)
    ml = workload.build_layer(cfg, max_tokens=8)
    try:
        L = cfg.n_layers
        ml.set_shared(L - 1, 0, oracle_blob(cfg, L - 1, cfg.E))
        wg, wu, wd = synth.expert_weights(cfg, 1, cfg.E)
        M._check("moe_requant_shared", M.moe_requant_shared(
            ml.ctx, 1, 0, M.MOE_SRC_F32, torch.from_numpy(wg).cuda(), torch.from_numpy(wu).cuda(),
            torch.from_numpy(wd).cuda(), None, None, None))
        torch.cuda.synchronize()
        for layer in range(L):
            assert np.array_equal(ml.read_shared(layer, 0), oracle_blob(cfg, layer, cfg.E)), layer
        for layer in range(L):
            ref = OracleLayer(cfg, layer)
            for T in (1, 5):
                x = synth.tokens(cfg, T=T, stream=20 + layer)
                got = ml.forward(torch.from_numpy(x).cuda(), layer).cpu().numpy()
                r_out, _, _, gk, gi = ref.forward(x)
                excluded, _ = flags(gk, gi)
                err = rel_err(got, r_out, ~excluded)
                log(f"{name} layer {layer} T={T}: max|d|/max|ref| = {err:.2e}")
                assert err <= REL_TOL
        assert ml.status()[0] == 0
    finally:
        ml.close()


@pytest.mark.parametrize("kind", ["f32", "bf16", "fp8"])
def test_requant_shared_int8(kind):
    """Checkpoint tensors on the device -> the int8 shared slot, byte for
    byte the oracle's blob of the decoded weights."""
    H, I = 512, 768
    ml = MoeLayer(H, I, 16, 2, 1, 1, oracle.W_INT4_ROW, n_slots=1, max_tokens=2,
                  shared_fmt=oracle.W_INT8_ROW)
    try:
        srcs = []
        for t, (O, In) in enumerate([(I, H), (I, H), (H, I)]):
            k = synth.key(951, 0, t)
            if kind == "fp8":
                srcs.append(synth.fp8_checkpoint(k, O, In, 0.02))
            elif kind == "bf16":
                srcs.append((synth.bf16_checkpoint(k, O, In, 0.02), None))
            else:
                srcs.append((synth.gauss(k, O * In, 0.02).reshape(O, In), None))

        def dev(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

        ml.requant_shared(0, 0, KINDS[kind], *[dev(w) for w, _ in srcs], *[dev(s) for _, s in srcs])
        want = oracle.pack_expert(oracle.W_INT8_ROW,
                                  *[oracle.decode_source(w, KINDS[kind], s) for w, s in srcs])
        assert np.array_equal(ml.read_shared(0, 0), want)
    finally:
        ml.close()


@pytest.mark.parametrize("path", ["gemm", "gemv"])
def test_many_tokens(path):
    """T = 300 with an int8 shared expert: through the grouped GEMM (the
    shared expert's tiles take int8 B operands) and, with the GEMM threshold
    raised, through the GEMVs (past their k-slice partial buffers' 16 and 64
    tokens, so the plan drops to fewer slices)."""
    cfg = synth.CONFIGS["int8_shared"]
    ml = workload.build_layer(cfg, max_tokens=300)
    ref = OracleLayer(cfg, 0)
    try:
        if path == "gemv":
            M._check("moe_set_gemm_min_tokens", M.moe_set_gemm_min_tokens(ml.ctx, 1 << 20))
        x = synth.tokens(cfg, T=300, stream=9)
        got = ml.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
        assert ml.status()[0] == 0
        r_out, _, _, gk, gi = ref.forward(x)
        excluded, _ = flags(gk, gi)
        err = rel_err(got, r_out, ~excluded)
        log(f"int8_shared T=300 ({path}): max|d|/max|ref| = {err:.2e}, {int(excluded.sum())} flagged")
        assert err <= REL_TOL
    finally:
        ml.close()


def test_glm_prefill_int8_shared():
    """GLM-shape prefill (T = 2048) with the shared expert in per-row int8
    through the grouped GEMM: routing of every token, and the outputs of
    tokens covering every occupied 32-row block of every expert's rows and of
    the shared expert's (whose tiles run the int8 operand path)."""
    cfg = synth.CONFIGS["glm_prefill_int8_shared"]
    log("building glm_prefill_int8_shared: 1 layer x 256 experts, T=2048")
    ml = workload.build_layer(cfg)
    try:
        x = synth.tokens(cfg, T=cfg.T)
        xd = torch.from_numpy(x).cuda()
        out = ml.forward(xd, 0).cpu().numpy()
        ids, w = ml.route(xd, 0)
        assert ml.status()[0] == 0
        ref = OracleLayer(cfg, 0)
        r_ids, r_w, _, _, gk, gi = ref.route(x)
        check_ids(ids.cpu().numpy(), r_ids, w.cpu().numpy(), r_w, gk, gi, "prefill int8 shared")
        excluded, _ = flags(gk, gi)
        sample, uncovered = block_sample(r_ids, cfg.E, excluded)
        assert uncovered <= 4
        r_out, _, _, _, _ = ref.forward(x[sample], workers=WORKERS)
        err = rel_err(out[sample], r_out)
        log(f"glm prefill, int8 shared: {len(sample)} tokens, max|d|/max|ref| = {err:.3e}")
        assert err <= REL_TOL
        assert np.isfinite(out).all()
    finally:
        ml.close()
        torch.cuda.empty_cache()


def test_graph_replay_int8_shared():
    """int8 shared experts under HIP-graph capture: every replay, with eager
    work and synchronisation between replays, equals the eager result."""
    cfg = synth.CONFIGS["int8_shared"]
    ml = workload.build_layer(cfg, max_tokens=8)
    try:
        xs = [torch.from_numpy(synth.tokens(cfg, T=T, stream=40 + T)).cuda() for T in (1, 4, 8)]
        eager = [ml.forward(x, 0).clone() for x in xs]
        outs = [torch.empty_like(x) for x in xs]
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        M.moe_set_stream(ml.ctx, cap.cuda_stream)
        try:
            with torch.cuda.graph(g, stream=cap):
                for x, o in zip(xs, outs):
                    M._check("moe_forward", M.moe_forward(ml.ctx, x, x.shape[0], 0, o))
        finally:
            M.moe_set_stream(ml.ctx, torch.cuda.current_stream().cuda_stream)
        for rep in range(4):
            for o in outs:
                o.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            for o, e in zip(outs, eager):
                assert torch.equal(o, e), rep
            other = ml.forward(torch.from_numpy(synth.tokens(cfg, T=3, stream=98)).cuda(), 0)
            torch.cuda.synchronize()
            assert torch.isfinite(other).all()
    finally:
        ml.close()
