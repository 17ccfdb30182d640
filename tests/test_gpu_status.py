"""Every status code of the C ABI produced by a real path on the GPU
(argument, size, slot, allocation, unsupported configuration, missing
expert, non-finite input and busy slot), each through the C ABI.  The
remaining code, MOE_E_HIP, is produced without a GPU (create on a machine
with no device, tests/test_abi.py)."""
import numpy as np
import pytest

import synth
from parity import OracleLayer, flags, log, rel_err, REL_TOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M, workload  # noqa: E402

CFG = synth.CONFIGS["tiny"]


@pytest.fixture(scope="module")
def layer():
    ml = workload.build_layer(CFG, max_tokens=128)
    yield ml
    ml.close()


def test_argument_size_slot_codes(layer):
    x = torch.zeros((2, CFG.H), device="cuda")
    assert M.moe_forward(layer.ctx, x, 0, 0, x) == M.MOE_E_ARG            # T = 0
    assert M.moe_forward(layer.ctx, x, 2, 0, x) == M.MOE_E_ARG            # x and out alias
    assert M.moe_forward(layer.ctx, x, 2, CFG.n_layers, x) == M.MOE_E_ARG  # layer out of range
    blob = np.zeros(layer.expert_bytes - 1, np.uint8)
    assert M.moe_load_expert(layer.ctx, 0, blob, blob.nbytes) == M.MOE_E_SIZE
    assert M.moe_load_expert(layer.ctx, 10 ** 6, blob, blob.nbytes) == M.MOE_E_SLOT
    assert M.moe_map_expert(layer.ctx, 0, 0, 10 ** 6) == M.MOE_E_SLOT


def test_nomem_and_unsupported():
    huge = M.make_config(6144, 2048, 256, 8, 1, 1, 1, 10 ** 6, 4)   # 18.9 TB of slots
    rc, h = M.moe_layer_create_rc(huge)
    assert rc == M.MOE_E_NOMEM and not h
    bad = M.make_config(512, 256, 300, 4, 1, 1, 1, 32, 4)            # 300 experts
    rc, h = M.moe_layer_create_rc(bad)
    assert rc == M.MOE_E_UNSUPPORTED and not h


def test_busy_slot(layer):
    img = np.zeros(layer.expert_bytes, np.uint8)
    # slot 0 holds (layer 0, expert 0) in the table: an asynchronous load is refused
    assert M.moe_load_image_async(layer.ctx, 0, img, img.nbytes) == M.MOE_E_BUSY


@pytest.mark.parametrize("T", [1, 4, 100])
def test_non_finite_input_is_reported(layer, T):
    """A NaN or an infinity in one row sets MOE_E_RANGE (small-T router and
    the large-T token statistics); the status clears, and the next forward
    on finite input is clean and matches the oracle."""
    x = synth.tokens(CFG, T=T, stream=300 + T)
    for bad in (np.nan, np.inf):
        xb = x.copy()
        xb[T // 2, 7] = bad
        layer.forward(torch.from_numpy(xb).cuda(), 0)
        rc, missing = layer.status()
        assert rc == M.MOE_E_RANGE and missing == [], (bad, rc)
        assert layer.status()[0] == M.MOE_OK          # cleared by the first call
    out = layer.forward(torch.from_numpy(x).cuda(), 0).cpu().numpy()
    assert layer.status()[0] == M.MOE_OK
    r_out, _, _, gk, gi = OracleLayer(CFG, 0).forward(x)
    excluded, _ = flags(gk, gi)
    err = rel_err(out, r_out, ~excluded)
    log(f"T={T} after the non-finite inputs: max|d|/max|ref| = {err:.2e}")
    assert err <= REL_TOL


def test_missing_expert_code(layer):
    x = synth.tokens(CFG, T=1, stream=401)
    r_ids = OracleLayer(CFG, 0).route(x)[0]
    victim = int(r_ids[0, 0])
    layer.map(0, victim, -1)
    try:
        layer.forward(torch.from_numpy(x).cuda(), 0)
        rc, missing = layer.status()
        assert rc == M.MOE_E_NOT_RESIDENT and missing == [victim]
    finally:
        layer.map(0, victim, victim)
    assert layer.status()[0] == M.MOE_OK
