"""GPU checks of the stand-alone steps through the C ABI: input generator,
int4 packers (bit-exact against the oracle), slot layout round trip,
bucketing (bit-exact against the oracle), argument errors."""
import numpy as np
import pytest

import oracle
import synth
from parity import log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M  # noqa: E402
from int4_weight_expert_amd.layer import MoeLayer  # noqa: E402


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_device_generator_matches_host():
    n = 1 << 20
    k = synth.key(5, 3, synth.T_GATE, 17)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.gpu_fill_gauss(out.data_ptr(), n, k, 0.02, 12345)
    torch.cuda.synchronize()
    host = synth.gauss(k, n, 0.02, 12345)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), host.view(np.uint32))


def _pack_rows_gpu(w):
    O, I = w.shape
    q = torch.empty((O, I // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty(O, dtype=torch.float32, device="cuda")
    assert M.moe_pack_int4_rows(dev(w), O, I, q, s) == 0
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _row_cases():
    yield "gauss", synth.gauss(synth.key(1, 0, synth.T_GATE, 0), 96 * 6144, 0.02).reshape(96, 6144)
    s = np.float32(2.0 ** -4)
    ties = np.tile(np.array([0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 7.0, 0.0], np.float32), (4, 8)) * s
    yield "ties", ties
    z = np.zeros((3, 256), np.float32)
    z[1, 7] = 1e-12                        # scale floor
    z[2] = -1.0                            # constant row
    yield "zero_floor_constant", z
    w = synth.gauss(synth.key(2, 0, synth.T_DOWN, 0), 64 * 2048, 1.0).reshape(64, 2048)
    w[::7] *= 1e4
    yield "wide_range", w.astype(np.float32)
    yield "odd_rows", synth.gauss(synth.key(3, 0, synth.T_UP, 0), 37 * 62, 0.5).reshape(37, 62)


@pytest.mark.parametrize("name,w", list(_row_cases()), ids=[c[0] for c in _row_cases()])
def test_pack_int4_rows_bit_exact(name, w):
    log(f"pack_int4_rows {name} {w.shape}")
    q, s = _pack_rows_gpu(w)
    rq, rs = oracle.pack_int4_row(w)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q, rq)


def _affine_cases():
    yield "gauss", synth.gauss(synth.key(4, 0, synth.T_GATE, 1), 64 * 2048, 0.02).reshape(64, 2048)
    c = np.full((4, 128), 0.3, np.float32)
    c[1, 64:] = np.linspace(-1, 1, 64)
    yield "constant_and_ramp", c
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(8, 256))
    codes[:, ::64], codes[:, 1::64] = 0, 15
    yield "exact_grid", (codes * 2.0 ** -6 - 0.25).astype(np.float32)


@pytest.mark.parametrize("name,w", list(_affine_cases()), ids=[c[0] for c in _affine_cases()])
def test_pack_affine_g64_bit_exact(name, w):
    log(f"pack_affine_g64 {name} {w.shape}")
    O, I = w.shape
    q = torch.empty((O, I // 2), dtype=torch.uint8, device="cuda")
    sm = torch.empty((O, I // 64, 2), dtype=torch.int16, device="cuda")
    assert M.moe_pack_affine_g64(dev(w), O, I, q, sm) == 0
    torch.cuda.synchronize()
    rq, rsm = oracle.pack_affine_g64(w)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(sm.cpu().numpy().view(np.uint16), rsm)


@pytest.mark.parametrize("fmt,H,I", [(1, 512, 256), (2, 2048, 512), (1, 6144, 2048)])
def test_slot_layout_round_trip_and_device_pack(fmt, H, I):
    log(f"slot round trip fmt={fmt} H={H} I={I}")
    cfg = synth.CONFIGS["tiny"].with_(H=H, I=I, fmt=fmt)
    ml = MoeLayer(H, I, 8, 2, 0, 1, fmt, n_slots=2, max_tokens=1)
    try:
        blob = oracle.pack_expert(fmt, *synth.expert_weights(cfg, 0, 3))
        ml.load_expert(0, blob)
        assert np.array_equal(ml.read_slot(0), blob)
        wg, wu, wd = (dev(a.ravel()) for a in synth.expert_weights(cfg, 0, 3))
        ml.pack_expert(1, wg, wu, wd)
        assert np.array_equal(ml.read_slot(1), blob)
    finally:
        ml.close()


def _bucket_gpu(ids, E):
    T, K = ids.shape
    d = dev(ids.astype(np.int32))
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * K, dtype=torch.int32, device="cuda")
    act = torch.empty(E, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    assert M.moe_bucket(d, T, K, E, cnt, off, perm, act, na) == 0
    torch.cuda.synchronize()
    n = int(na.item())
    return cnt.cpu().numpy(), off.cpu().numpy(), perm.cpu().numpy(), act.cpu().numpy()[:n]


def _bucket_cases():
    rng = np.random.default_rng(1)
    yield "one", np.array([[5]]), 256
    yield "all_same", np.zeros((100, 1), int), 8
    yield "decode_k8", np.stack([rng.permutation(256)[:8] for _ in range(1)]), 256
    yield "verify_8x8", np.stack([rng.permutation(256)[:8] for _ in range(8)]), 256
    skew = np.minimum(rng.zipf(1.3, size=(2048, 8)) - 1, 255)
    yield "prefill_skewed_2048x8", skew, 256
    yield "max_65536", rng.integers(0, 256, size=(8192, 8)), 256
    yield "ragged_1000x3_e7", rng.integers(0, 7, size=(1000, 3)), 7


@pytest.mark.parametrize("name,ids,E", list(_bucket_cases()), ids=[c[0] for c in _bucket_cases()])
def test_bucket_bit_exact(name, ids, E):
    log(f"bucket {name} {ids.shape} E={E}")
    got = _bucket_gpu(ids, E)
    ref = oracle.bucket(ids.astype(np.int32), E)
    for g, r, what in zip(got, ref, ("cnt", "off", "perm", "active")):
        assert np.array_equal(g, r), what


def test_argument_errors():
    ml = MoeLayer(512, 256, 32, 4, 1, 2, 1, n_slots=4, max_tokens=4)
    try:
        x = torch.zeros((4, 512), device="cuda")
        out = torch.zeros((4, 512), device="cuda")
        c = ml.ctx
        assert M.moe_forward(c, x, 0, 0, out) == M.MOE_E_ARG
        assert M.moe_forward(c, x, 5, 0, out) == M.MOE_E_ARG
        assert M.moe_forward(c, x, 1, 2, out) == M.MOE_E_ARG
        assert M.moe_forward(c, x, 4, 0, x) == M.MOE_E_ARG              # aliasing
        assert M.moe_forward(c, x, 4, 0, x[1:]) == M.MOE_E_ARG           # partial overlap
        blob = np.zeros(ml.expert_bytes + 1, np.uint8)
        assert M.moe_load_expert(c, 0, blob, blob.nbytes) == M.MOE_E_SIZE
        assert M.moe_load_expert(c, 4, blob, ml.expert_bytes) == M.MOE_E_SLOT
        assert M.moe_map_expert(c, 0, 32, 0) == M.MOE_E_ARG
        assert M.moe_map_expert(c, 0, 0, 9) == M.MOE_E_SLOT
        assert M.moe_set_shared(c, 0, 1, blob, ml.expert_bytes) == M.MOE_E_ARG
        rc, _ = ml.status()
        assert rc == 0
    finally:
        ml.close()
    # K = 4 above the 2 experts of the one kept group
    cfg = M.make_config(512, 256, 32, 4, 1, 1, 1, 4, 4, n_group=16, topk_group=1)
    rc, h = M.moe_layer_create_rc(cfg)
    assert rc == M.MOE_E_UNSUPPORTED and not h
