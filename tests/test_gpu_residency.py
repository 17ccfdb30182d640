"""Expert residency through the C ABI (Edge0 write-up §十四 staged and
whole-layer paths; "惊呆了！…" §13 one read per expert): slot images loaded
asynchronously from pinned host memory, whole-layer loads, the staged
executor's sticky slots, and the ordering of loads against forwards that
may still read a slot.  Outputs follow the usual 2e-3 rule against the
oracle; bytes are exact."""
import numpy as np
import pytest

import oracle
import synth
from parity import OracleLayer, check_ids, flags, log, oracle_blob, rel_err, REL_TOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_expert_amd import moe as M  # noqa: E402
from int4_weight_expert_amd.layer import MoeLayer  # noqa: E402

CFG = synth.CONFIGS["tiny"]


def new_layer(cfg, n_slots, n_layers=1, max_tokens=64):
    ml = MoeLayer(cfg.H, cfg.I, cfg.E, cfg.K, cfg.n_shared, n_layers, cfg.fmt, n_slots=n_slots,
                  max_tokens=max_tokens, routed_scale=cfg.routed_scale, norm_topk=cfg.norm_topk)
    for l in range(n_layers):
        ml.set_router(l, synth.router_weight(cfg, l), synth.router_bias(cfg, l))
        for s in range(cfg.n_shared):
            ml.set_shared(l, s, oracle_blob(cfg, l, cfg.E + s))
    return ml


def pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.empty(a.nbytes, dtype=torch.uint8, pin_memory=True)
    t.numpy()[:] = a.reshape(-1).view(np.uint8)
    return t


@pytest.fixture(scope="module")
def blobs():
    return {e: oracle_blob(CFG, 0, e) for e in range(CFG.E)}


def check_forward(ml, ref, x, layer=0, out=None):
    xd = torch.from_numpy(x).cuda()
    got = ml.forward(xd, layer).cpu().numpy() if out is None else out
    r_out, r_ids, r_w, gk, gi = ref.forward(x)
    excluded, _ = flags(gk, gi)
    err = rel_err(got, r_out, ~excluded)
    assert err <= REL_TOL, err
    return err


def test_image_round_trip(blobs):
    ml = new_layer(CFG, 4)
    try:
        for slot, e in enumerate([0, 5, 17, 31]):
            ml.load_image_async(slot, pinned(ml.image(blobs[e])))
        for slot, e in enumerate([0, 5, 17, 31]):
            assert np.array_equal(ml.read_slot(slot), blobs[e])
    finally:
        ml.close()


def test_whole_layer_load_then_forward(blobs):
    ml = new_layer(CFG, CFG.E)
    try:
        images = np.concatenate([ml.image(blobs[e]) for e in range(CFG.E)])
        ml.load_layer_async(0, 0, CFG.E, pinned(images))
        ref = OracleLayer(CFG, 0)
        for T in (1, 7, 64):
            log(f"whole-layer forward T={T}")
            check_forward(ml, ref, synth.tokens(CFG, T=T, stream=40 + T))
        assert ml.status()[0] == 0
    finally:
        ml.close()


def test_async_map_without_sync(blobs):
    ml = new_layer(CFG, CFG.E)
    try:
        for e in range(CFG.E):
            ml.load_image_async(e, pinned(ml.image(blobs[e])))
        ml.map_async(0, list(range(CFG.E)), list(range(CFG.E)))
        check_forward(ml, OracleLayer(CFG, 0), synth.tokens(CFG, T=16, stream=3))
    finally:
        ml.close()


def expected_plan(held, used, want):
    """The staged executor's slot rule, written out: held wanted experts stay;
    the rest take empty slots (ascending), then the least recently wanted."""
    slot_of, n = {}, 0
    for w in want:
        if w in held:
            slot_of[w] = held.index(w)
    free = sorted((j for j in range(len(held)) if j not in slot_of.values()),
                  key=lambda j: (held[j] >= 0, used[j], j))
    for w in want:
        if w not in slot_of:
            slot_of[w] = free[n]
            n += 1
    return n, slot_of


def test_staged_steps_are_sticky(blobs):
    """Each step stages the experts the step's tokens route to; experts
    already staged are not loaded again."""
    P = 12
    ml = new_layer(CFG, P)
    ref = OracleLayer(CFG, 0)
    images = {e: pinned(ml.image(blobs[e])) for e in range(CFG.E)}
    try:
        ml.set_staging(0, P)
        held, used = [-1] * P, [-1] * P
        for step in range(10):
            T = 1 + step % 3
            x = synth.tokens(CFG, T=T, stream=100 + step % 5)   # batches repeat every 5 steps
            ids, *_ = ref.route(x)
            want = sorted(set(int(v) for v in np.ravel(ids)))
            n = ml.stage(0, want, [images[e] for e in want])
            r_n, slot_of = expected_plan(held, used, want)
            assert n == r_n, (step, n, r_n)
            for w, j in slot_of.items():
                held[j], used[j] = w, step
            log(f"step {step}: T={T} want {len(want)} loaded {n}")
            check_forward(ml, ref, x)
        assert ml.stage(0, want, [None] * len(want)) == 0   # same set again: nothing to load
    finally:
        ml.close()


def test_slot_reuse_waits_for_earlier_forward(blobs):
    """Forward A is enqueued on staged experts; the next stage evicts some of
    them (every staged slot is full) for set B before A has run.  A must
    still see its experts, B its own."""
    ref = OracleLayer(CFG, 0)
    xa = synth.tokens(CFG, T=4, stream=7)
    ids_a, *_ = ref.route(xa)
    set_a = sorted(set(int(v) for v in np.ravel(ids_a)))
    xb = None
    for s in range(200):   # a one-token batch that needs an expert outside set A
        x = synth.tokens(CFG, T=1, stream=1000 + s)
        ib, *_ = ref.route(x)
        b = sorted(set(int(v) for v in np.ravel(ib)))
        if set(b) - set(set_a):
            xb, set_b = x, b
            break
    assert xb is not None
    P = len(set_a)
    ml = new_layer(CFG, P)
    images = {e: pinned(ml.image(blobs[e])) for e in range(CFG.E)}
    try:
        ml.set_staging(0, P)
        ml.stage(0, set_a, [images[e] for e in set_a])
        xad, xbd = torch.from_numpy(xa).cuda(), torch.from_numpy(xb).cuda()
        outs_a = [ml.forward(xad, 0) for _ in range(6)]      # queued, not synchronised
        n = ml.stage(0, set_b, [images[e] for e in set_b])
        assert n == len(set(set_b) - set(set_a)) > 0
        out_b = ml.forward(xbd, 0)
        torch.cuda.synchronize()
        for o in outs_a:
            check_forward(ml, ref, xa, out=o.cpu().numpy())
        check_forward(ml, ref, xb, out=out_b.cpu().numpy())
    finally:
        ml.close()


def test_busy_and_argument_errors(blobs):
    ml = new_layer(CFG, 2)
    try:
        img = pinned(ml.image(blobs[0]))
        ml.load_image_async(0, img)
        ml.map(0, 0, 0)
        assert M.moe_load_image_async(ml.ctx, 0, img, img.numel()) == M.MOE_E_BUSY
        assert M.moe_load_image_async(ml.ctx, 2, img, img.numel()) == M.MOE_E_SLOT
        assert M.moe_load_image_async(ml.ctx, 1, img, img.numel() - 1) == M.MOE_E_SIZE
        assert M.moe_stage_experts(ml.ctx, 0, [1], [img])[0] == M.MOE_E_ARG   # staging not set
        assert M.moe_set_staging(ml.ctx, 1, 2) == M.MOE_E_SLOT
        assert M.moe_set_staging(ml.ctx, 1, 1) == M.MOE_OK
        assert M.moe_stage_experts(ml.ctx, 0, [1, 2], [img, img])[0] == M.MOE_E_ARG  # > per_layer
        assert M.moe_stage_experts(ml.ctx, 0, [3], [None])[0] == M.MOE_E_ARG        # no image
        assert M.moe_load_layer_async(ml.ctx, 0, 0, 2, img, 2 * img.numel()) == M.MOE_E_BUSY
        ml.sync_copies()
        assert np.array_equal(ml.read_slot(0), blobs[0])
    finally:
        ml.close()
