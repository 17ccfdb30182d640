"""The converter step on the GPU ([GLM-C] §06): checkpoint tensors (fp32,
bf16, FP8 E4M3 with 128 x 128 block inverse scales) requantised to int4 by
the library, and the converter's offset-binary container imported into a
slot.  Codes and scales are integer/byte results of fp32 decisions taken in
the pages' precision, so they must equal the oracle's bit for bit; layer
outputs built from them follow the usual 2e-3 rule."""
import numpy as np
import pytest

import oracle
import synth
from parity import log, rel_err, REL_TOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M  # noqa: E402
from int4_weight_expert_amd.layer import MoeLayer  # noqa: E402

KINDS = {"f32": oracle.SRC_F32, "bf16": oracle.SRC_BF16, "fp8": oracle.SRC_FP8_E4M3}
ROW, AFF = oracle.W_INT4_ROW, oracle.W_INT4_AFFINE_G64


def source(kind, O, I, k, sigma=0.02):
    """(host array in the source kind, inverse scales or None)."""
    if kind == "fp8":
        return synth.fp8_checkpoint(k, O, I, sigma)
    if kind == "bf16":
        return synth.bf16_checkpoint(k, O, I, sigma), None
    return synth.gauss(k, O * I, sigma).reshape(O, I), None


def dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def plant_degenerate_rows(kind, w):
    """Row 0 all zero (the 1e-8 floor), row 1 a single nonzero."""
    w = w.copy()
    w[0] = 0
    w[1] = 0
    w[1, w.shape[1] // 3] = w.dtype.type(0x38) if kind == "fp8" else (
        np.uint16(0x3F80) if kind == "bf16" else np.float32(1.0))
    return w


def gpu_rows(kind, w, sinv):
    O, I = w.shape
    q = torch.empty((O, I // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty(O, dtype=torch.float32, device="cuda")
    M._check("moe_requant_int4_rows",
             M.moe_requant_int4_rows(dev(w), KINDS[kind], dev(sinv), O, I, q, s, 0))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


# shapes: the wave-per-row kernel (I % 32 == 0, I <= 8192) and the generic one
SHAPES = [(257, 2048), (64, 8192), (130, 32), (300, 1040), (33, 8224), (7, 6)]


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("O,I", SHAPES)
def test_requant_rows_match_oracle(kind, O, I):
    log(f"requant rows {kind} {O}x{I}")
    w, sinv = source(kind, O, I, synth.key(900, 0, O, I))
    w = plant_degenerate_rows(kind, w) if O > 2 else w
    q, s = gpu_rows(kind, w, sinv)
    rq, rs = oracle.requant_int4_rows(w, KINDS[kind], sinv)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q, rq)


@pytest.mark.parametrize("I", [32, 30])
def test_fp8_every_code(I):
    """Row c holds FP8 code c then zeros: its scale is |code| / 7 and its
    first code +-7, so every non-NaN code's decode is visible."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    w = np.zeros((len(codes), I), dtype=np.uint8)
    w[:, 0] = codes
    sinv = np.ones(((len(codes) + 127) // 128, 1), dtype=np.float32)
    q, s = gpu_rows("fp8", w, sinv)
    rq, rs = oracle.requant_int4_rows(w, oracle.SRC_FP8_E4M3, sinv)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q, rq)


@pytest.mark.parametrize("I", [256, 250])
def test_requant_ties_and_near_ties(I):
    """w / s at exact half-integers (ties to even) and one ulp either side
    of them, where the fast reciprocal path must defer to the exact
    quotient."""
    rng = np.random.default_rng(4)
    O = 96
    s = np.float32(2.0 ** -4)
    k = rng.integers(-7, 7, size=(O, I)).astype(np.float32) + np.float32(0.5)
    w = (k * s).astype(np.float32)
    nudge = rng.integers(-1, 2, size=(O, I))
    w = np.where(nudge > 0, np.nextafter(w, np.float32(np.inf)),
                 np.where(nudge < 0, np.nextafter(w, np.float32(-np.inf)), w)).astype(np.float32)
    w[:, 5] = 7 * s
    q, sc = gpu_rows("f32", w, None)
    rq, rs = oracle.requant_int4_rows(w, oracle.SRC_F32, None)
    assert np.array_equal(sc, rs) and np.array_equal(q, rq)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("O,I", [(130, 256), (64, 1024)])
def test_requant_affine_match_oracle(kind, O, I):
    w, sinv = source(kind, O, I, synth.key(901, 0, O, I))
    q = torch.empty((O, I // 2), dtype=torch.uint8, device="cuda")
    sm = torch.empty((O, I // 64, 2), dtype=torch.int16, device="cuda")
    M._check("moe_requant_affine_g64",
             M.moe_requant_affine_g64(dev(w), KINDS[kind], dev(sinv), O, I, q, sm, 0))
    torch.cuda.synchronize()
    rq, rsm = oracle.pack_affine_g64(oracle.decode_source(w, KINDS[kind], sinv))
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sm.cpu().numpy().view(np.uint16).reshape(rsm.shape), rsm)


def expert_sources(kind, H, I, seed, e):
    return [source(kind, O, In, synth.key(seed, 0, t, e))
            for t, (O, In) in enumerate([(I, H), (I, H), (H, I)])]


def oracle_expert_blob(fmt, kind, srcs):
    return oracle.pack_expert(fmt, *[oracle.decode_source(w, KINDS[kind], si) for w, si in srcs])


@pytest.mark.parametrize("fmt,H,I,kind", [(ROW, 512, 256, "fp8"), (ROW, 6144, 2048, "fp8"),
                                          (ROW, 2048, 512, "bf16"), (AFF, 2048, 512, "fp8"),
                                          (ROW, 512, 256, "f32")])
def test_requant_expert_into_slot(fmt, H, I, kind):
    log(f"requant expert fmt={fmt} H={H} I={I} {kind}")
    ml = MoeLayer(H, I, 8, 2, 0, 1, fmt, n_slots=2, max_tokens=4)
    try:
        for slot in range(2):
            srcs = expert_sources(kind, H, I, 902 + slot, slot)
            d = [(dev(w), dev(si)) for w, si in srcs]
            ml.requant_expert(slot, KINDS[kind], d[0][0], d[1][0], d[2][0], d[0][1], d[1][1],
                              d[2][1])
            torch.cuda.synchronize()
            assert np.array_equal(ml.read_slot(slot), oracle_expert_blob(fmt, kind, srcs))
    finally:
        ml.close()


def test_requant_layer_forward():
    """A layer whose routed and shared experts all come from FP8 sources."""
    cfg = synth.CONFIGS["tiny"]
    H, I, E = cfg.H, cfg.I, cfg.E
    ml = MoeLayer(H, I, E, cfg.K, cfg.n_shared, 1, cfg.fmt, n_slots=E, max_tokens=64)
    try:
        ml.set_router(0, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0))
        blobs, shared = [], []
        for e in range(E + cfg.n_shared):
            srcs = expert_sources("fp8", H, I, 903, e)
            d = [(dev(w), dev(si)) for w, si in srcs]
            args = (oracle.SRC_FP8_E4M3, d[0][0], d[1][0], d[2][0], d[0][1], d[1][1], d[2][1])
            if e < E:
                ml.requant_expert(e, *args)
                ml.map(0, e, e)
                blobs.append(oracle_expert_blob(cfg.fmt, "fp8", srcs))
            else:
                ml.requant_shared(0, e - E, *args)
                shared.append(oracle_expert_blob(cfg.fmt, "fp8", srcs))
        torch.cuda.synchronize()
        for T in (1, 4, 64):
            x = synth.tokens(cfg, T=T, stream=T)
            out = ml.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
            ref, _, _ = oracle.moe_layer(x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0),
                                         cfg.K, cfg.fmt, I, blobs, shared, cfg.routed_scale,
                                         cfg.norm_topk)
            err = rel_err(out, ref, ~near_tie(cfg, x))
            log(f"  T={T} max|d|/max|ref| = {err:.3e}")
            assert err <= REL_TOL
    finally:
        ml.close()


def near_tie(cfg, x):
    """Tokens whose routing has several correct answers within rounding."""
    _, _, _, _, gk, _ = oracle.route(x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0),
                                     cfg.K, cfg.routed_scale, cfg.norm_topk)
    return np.asarray(gk) < 1e-4


def container_expert(H, I, seed, e, plant_min=True):
    """The converter's container for one expert, with some codes set to -8
    (nibble 0), which the container allows though the quantiser never makes it."""
    out = []
    for t, (O, In) in enumerate([(I, H), (I, H), (H, I)]):
        w = synth.gauss(synth.key(seed, 0, t, e), O * In, 0.02).reshape(O, In)
        q, s = oracle.convert_int4_container(w)
        if plant_min:
            q[::7, ::5] &= 0xF0
        out.append((q, s))
    return out


def container_blob(parts):
    qs = [q ^ 0x88 for q, _ in parts]
    return np.concatenate([a.reshape(-1).view(np.uint8) for a in qs] +
                          [s.view(np.uint8) for _, s in parts])


@pytest.mark.parametrize("host", [True, False])
def test_import_container(host):
    cfg = synth.CONFIGS["tiny"]
    H, I, E = cfg.H, cfg.I, cfg.E
    ml = MoeLayer(H, I, E, cfg.K, cfg.n_shared, 1, cfg.fmt, n_slots=E, max_tokens=64)
    try:
        ml.set_router(0, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0))
        blobs, shared = [], []
        for e in range(E + cfg.n_shared):
            parts = container_expert(H, I, 904, e)
            args = [p[0] for p in parts] + [p[1] for p in parts]
            if not host:
                args = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in args]
            if e < E:
                ml.import_expert(e, *args)
                ml.map(0, e, e)
                blobs.append(container_blob(parts))
                assert np.array_equal(ml.read_slot(e), blobs[-1])
            else:
                ml.import_shared(0, e - E, *args)
                shared.append(container_blob(parts))
        for T in (1, 5, 64):
            x = synth.tokens(cfg, T=T, stream=T)
            out = ml.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
            ref, _, _ = oracle.moe_layer(x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0),
                                         cfg.K, cfg.fmt, I, blobs, shared, cfg.routed_scale,
                                         cfg.norm_topk)
            err = rel_err(out, ref, ~near_tie(cfg, x))
            log(f"  import T={T} max|d|/max|ref| = {err:.3e}")
            assert err <= REL_TOL
    finally:
        ml.close()


def test_requant_and_import_reject_bad_arguments():
    ml = MoeLayer(512, 256, 8, 2, 0, 1, ROW, n_slots=1, max_tokens=4)
    ma = MoeLayer(512, 256, 8, 2, 0, 1, AFF, n_slots=1, max_tokens=4)
    try:
        w = torch.zeros(256 * 512, dtype=torch.uint8, device="cuda")
        assert M.moe_requant_expert(ml.ctx, 0, 3, w, w, w) == M.MOE_E_ARG
        assert M.moe_requant_expert(ml.ctx, 0, oracle.SRC_FP8_E4M3, w, w, w) == M.MOE_E_ARG
        assert M.moe_requant_expert(ml.ctx, 1, oracle.SRC_BF16, w, w, w) == M.MOE_E_SLOT
        s = torch.zeros(512, dtype=torch.float32, device="cuda")
        assert M.moe_import_expert(ma.ctx, 0, w, w, w, s, s, s) == M.MOE_E_UNSUPPORTED
        assert M.moe_import_expert(ml.ctx, 0, w, None, w, s, s, s) == M.MOE_E_ARG
        q = torch.empty(64, dtype=torch.uint8, device="cuda")
        assert M.moe_requant_int4_rows(w, 2, None, 4, 32, q, s, 0) == M.MOE_E_ARG
        assert M.moe_requant_int4_rows(w, 0, None, 4, 31, q, s, 0) == M.MOE_E_ARG
    finally:
        ml.close()
        ma.close()
