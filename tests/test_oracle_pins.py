"""Pins of the CPU oracle to facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
printed on the pages (tests/golden), closed forms, exact special cases,
invariants and brute force on tiny inputs.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ROW, AFF = oracle.W_INT4_ROW, oracle.W_INT4_AFFINE_G64


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


# ---------------------------------------------------------------------------
# sizes printed on the pages
# ---------------------------------------------------------------------------

def test_glm_expert_bytes_match_hot_tier_figures():
    g = _golden("expert_sizes.txt")
    b = oracle.blob_bytes(ROW, 6144, 2048)
    assert b == 3 * 6144 * 2048 // 2 + 4 * (2048 + 2048 + 6144)
    assert round(b * int(g["glm_hot_tier_experts"]) / 1e9, 2) == float(g["glm_hot_tier_gb"])
    assert round(b * int(g["glm_device_experts"]) / 1e9, 2) == float(g["glm_device_gb"])
    assert round(b / 1e6, 1) == float(g["glm_expert_mb"])


def test_edge0_expert_bytes_match_byte_account():
    g = _golden("expert_sizes.txt")
    b = oracle.blob_bytes(AFF, 2048, 512)
    assert round(b / 1e6, 2) == float(g["edge0_expert_mb"])
    assert round(256 * b / 1e6) == pytest.approx(float(g["edge0_layer_mb"]), abs=1)
    assert round(40 * 256 * b / 1e9, 1) == float(g["edge0_total_gb"])
    assert round(40 * 4 * b / 1e6) == pytest.approx(float(g["edge0_tok_mb"]), abs=1)


def test_mac_counts_match_dataflow_page():
    """The oracle's own expert counts its multiply-adds: with every code +1,
    every scale 1 and x = 1, a gate (or up) row sums exactly its H inputs, so
    g = u = H and h = silu(H) * H = H^2 (exp(-6144) underflows to 0); a down
    row sums its I values of h, so y = I * h.  Rows times inputs per row give
    the MACs of one token through one expert."""
    g = _golden("expert_sizes.txt")
    H, I, E = 6144, 2048, 256
    nb = oracle.blob_bytes(ROW, H, I)
    blob = np.full(nb, 0x11, dtype=np.uint8)            # two +1 codes per byte
    blob[3 * H * I // 2:] = np.ones(2 * I + H, dtype=np.float32).view(np.uint8)
    y, h = oracle.expert(ROW, H, I, blob, np.ones(H, dtype=np.float32))
    assert h.shape == (I,) and y.shape == (H,)
    per_gate_row = np.sqrt(h.astype(np.float64))         # g = u = inputs per row
    per_down_row = y.astype(np.float64) / float(h[0])   # inputs per down row
    assert np.all(per_gate_row == H) and np.all(per_down_row == I)
    macs = int(per_gate_row.sum() * 2 + per_down_row.sum())
    assert macs == 3 * H * I
    assert round(macs / 1e6, 1) == float(g["glm_expert_mmacs"])
    assert round(8 * macs / 1e6) == float(g["glm_routed8_mmacs"])
    # the router: one logit per expert, each a dot product over H inputs
    _, _, logits, _, _, _ = oracle.route(np.ones((1, H), np.float32),
                                         np.ones((E, H), np.float32), np.zeros(E, np.float32), 8)
    assert logits.shape == (1, E) and np.all(logits == H)
    assert round(logits.size * float(logits[0, 0]) / 1e6, 1) == float(g["glm_router_mmacs"])


# ---------------------------------------------------------------------------
# O1 / O3: per-row int4 pack and unpack
# ---------------------------------------------------------------------------

def test_page_container_example_decodes():
    g = _golden("int4_container_example.txt")
    raw = np.array([int(b, 16) for b in g["bytes_offset_binary"].split()], dtype=np.uint8)
    want_lo = [int(v) for v in g["low_nibble_codes"].split()]
    assert int(g["nbytes"]) * 2 // int(g["rows"]) == 6144
    # offset-binary (q + 8) -> two's complement nibbles: flip each nibble's top bit
    twos = (raw ^ 0x88).reshape(1, -1)
    codes = oracle.unpack_int4_row(twos, 16)[0]
    assert list(codes[0::2]) == want_lo
    # the high nibbles decode by the same rule (q = nibble - 8 in the page's encoding)
    assert list(codes[1::2]) == [int(b >> 4) - 8 for b in raw]


def test_nibble_order_and_twos_complement():
    s = 2.0 ** -4            # amax = 7 s so s is reproduced exactly
    row = np.array([[1, 0, 0, 0, 7, 0], [0, 1, 0, 0, 7, 0], [-1, 0, 0, 0, 7, 0],
                    [0, -7, 3, -3, 7, 0]], dtype=np.float32) * s
    q, sc = oracle.pack_int4_row(row)
    assert np.all(sc == np.float32(s))
    assert list(q[0]) == [0x01, 0x00, 0x07]
    assert list(q[1]) == [0x10, 0x00, 0x07]
    assert list(q[2]) == [0x0F, 0x00, 0x07]
    assert list(q[3]) == [0x90, 0xD3, 0x07]


def test_round_half_to_even():
    s = 2.0 ** -4            # 0.4375 / 7 == 0.0625 exactly
    w = np.array([[0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 7.0, 0.0]], dtype=np.float32) * s
    q, sc = oracle.pack_int4_row(w)
    assert sc[0] == np.float32(0.0625)
    codes = oracle.unpack_int4_row(q, 8)[0]
    # half-to-even; rounding half away from zero would give 1, 2, 3, -3, 4, -1
    assert list(codes) == [0, 2, 2, -2, 4, 0, 7, 0]


def test_every_byte_round_trips():
    s = 2.0 ** -5
    for b in range(256):
        lo, hi = b & 0xF, b >> 4
        if lo == 8 or hi == 8:      # code -8 is never produced (clamp [-7, 7])
            continue
        ql = lo - 16 if lo >= 8 else lo
        qh = hi - 16 if hi >= 8 else hi
        w = np.array([[ql, qh, 7, 0]], dtype=np.float32) * np.float32(s)
        q, sc = oracle.pack_int4_row(w)
        assert q[0, 0] == b and q[0, 1] == 0x07 and sc[0] == np.float32(s)


def test_pack_error_bound_and_code_range():
    w = synth.gauss(synth.key(7, 0, synth.T_GATE, 0), 64 * 512, 0.02).reshape(64, 512)
    w[3] *= 1e3
    w[5, :] = 0.0
    q, s = oracle.pack_int4_row(w)
    codes = oracle.unpack_int4_row(q, 512).astype(np.float64)
    assert codes.min() >= -7 and codes.max() <= 7
    amax = np.abs(w.astype(np.float64)).max(axis=1)
    for o in range(64):
        if o == 5:
            assert s[o] == np.float32(1e-8) and not codes[o].any()
            continue
        assert s[o] == np.float32(np.float32(amax[o]) / np.float32(7.0))
        err = np.abs(w[o].astype(np.float64) - codes[o] * float(s[o]))
        assert err.max() <= 0.5 * float(s[o]) * (1 + 1e-6)
        assert np.abs(codes[o]).max() == 7
    deq = oracle.dequant_int4_row(q, s, 512)
    assert np.array_equal(deq, codes * s.astype(np.float64)[:, None])


def test_odd_width_pads_high_nibble():
    w = np.array([[7, -7, 1]], dtype=np.float32)
    q, _ = oracle.pack_int4_row(w)
    assert q.shape == (1, 2) and q[0, 1] == 0x01


# ---------------------------------------------------------------------------
# O2 / O3: affine int4, group size 64
# ---------------------------------------------------------------------------

def test_affine_exact_grid_recovers_codes():
    rng = np.random.default_rng(3)
    O, I = 4, 128
    sc, mn = 2.0 ** -6, -0.25
    codes = rng.integers(0, 16, size=(O, I))
    codes[:, ::64] = 0
    codes[:, 1::64] = 15
    w = (codes * sc + mn).astype(np.float32)
    q, scmn = oracle.pack_affine_g64(w)
    assert np.all(scmn[..., 0] == 0x3C80)          # bf16 of 2^-6
    assert np.all(scmn[..., 1] == 0xBE80)          # bf16 of -0.25
    deq = oracle.dequant_affine_g64(q, scmn, I)
    assert np.array_equal(deq, w.astype(np.float64))
    lo = q & 0xF
    assert np.array_equal(lo, codes[:, 0::2])
    assert np.array_equal(q >> 4, codes[:, 1::2])


def test_affine_constant_group():
    w = np.full((2, 64), 0.3, dtype=np.float32)
    q, scmn = oracle.pack_affine_g64(w)
    assert not q.any() and np.all(scmn[..., 0] == 0)
    deq = oracle.dequant_affine_g64(q, scmn, 64)
    assert np.all(deq == oracle.bf16_round(0.3))


def test_affine_error_bound():
    w = synth.gauss(synth.key(9, 0, synth.T_DOWN, 0), 32 * 512, 0.02).reshape(32, 512)
    q, scmn = oracle.pack_affine_g64(w)
    deq = oracle.dequant_affine_g64(q, scmn, 512)
    for o in range(32):
        for g in range(8):
            seg = w[o, g * 64:(g + 1) * 64].astype(np.float64)
            s = oracle.bf16_round(float(np.float32(seg.max() - seg.min()) / np.float32(15)))
            m = oracle.bf16_round(float(seg.min()))
            # rounding of the code, plus what bf16 rounding of min and scale moves
            bound = 0.5 * s + abs(m - seg.min()) + 15 * abs(s - (seg.max() - seg.min()) / 15)
            assert np.abs(seg - deq[o, g * 64:(g + 1) * 64]).max() <= bound * (1 + 1e-6)


# ---------------------------------------------------------------------------
# O4: router
# ---------------------------------------------------------------------------

def _route_by_bias(bias, K):
    """x = 0 makes every logit 0 and every sigmoid exactly 0.5, so the
    selection score is 0.5 + bias."""
    E = len(bias)
    x = np.zeros((1, 8), dtype=np.float32)
    W = np.zeros((E, 8), dtype=np.float32)
    return oracle.route(x, W, np.asarray(bias, dtype=np.float32), K)


def test_topk_equals_brute_force_sort_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(300):
        E = int(rng.integers(1, 13))
        K = int(rng.integers(1, E + 1))
        bias = rng.integers(-3, 4, size=E).astype(np.float32) / 4   # many ties
        ids, wts, logits, sig, gk, gi = _route_by_bias(bias, K)
        c = [0.5 + float(b) for b in bias]
        want = sorted(range(E), key=lambda e: (-c[e], e))[:K]
        assert list(ids[0]) == want
        assert np.all(sig == 0.5) and np.all(logits == 0)
        assert np.allclose(wts[0], 2.5 / K, rtol=0, atol=1e-6)


def test_identical_scores_pick_lowest_ids():
    ids, *_ = _route_by_bias(np.zeros(16), 5)
    assert list(ids[0]) == [0, 1, 2, 3, 4]


def test_router_logits_one_hot_rows_and_sigmoid_symmetry():
    H, E = 16, 16
    x = (np.arange(H, dtype=np.float32) - 7.5).reshape(1, H) / 4
    W = np.eye(E, H, dtype=np.float32)
    W2 = -W
    b = np.zeros(E, dtype=np.float32)
    _, _, lg, sg, _, _ = oracle.route(x, W, b, 4)
    _, _, lg2, sg2, _, _ = oracle.route(x, W2, b, 4)
    assert np.array_equal(lg[0], x[0])
    # sigmoid(-z) = 1 - sigmoid(z); sigmoid(0) = 1/2; monotone increasing
    assert np.allclose(sg[0] + sg2[0], 1.0, atol=1e-7)
    assert np.all(np.diff(sg[0]) > 0)


def test_weights_renormalised_to_routed_scale():
    cfg = synth.CONFIGS["tiny"]
    W = synth.router_weight(cfg, 0)
    b = synth.router_bias(cfg, 0)
    x = synth.tokens(cfg, T=16)
    ids, wts, lg, sg, gk, gi = oracle.route(x, W, b, 4)
    assert np.allclose(wts.sum(axis=1), 2.5, atol=4 * 2.5 * 2 ** -23)
    for t in range(16):
        s = sg[t, ids[t]].astype(np.float64)
        assert np.allclose(wts[t], 2.5 * s / s.sum(), rtol=1e-7)
    # K = E: the weights are 2.5 * sigma / sum(sigma) over all experts
    ids, wts, lg, sg, gk, gi = oracle.route(x[:2], W, b, cfg.E)
    for t in range(2):
        order = np.argsort(ids[t])
        assert np.allclose(wts[t][order], 2.5 * sg[t] / sg[t].astype(np.float64).sum(),
                           rtol=1e-6)
        assert gk[t] == np.inf
    # no renormalisation: weight = 2.5 * sigma
    ids, wts, lg, sg, gk, gi = oracle.route(x, W, b, 4, norm_topk=0)
    for t in range(16):
        assert np.allclose(wts[t], 2.5 * sg[t, ids[t]], rtol=1e-7)


def test_router_permutation_equivariance():
    cfg = synth.CONFIGS["tiny"]
    W = synth.router_weight(cfg, 0)
    b = synth.router_bias(cfg, 0)
    x = synth.tokens(cfg, T=8)
    ids, wts, *_ = oracle.route(x, W, b, 4)
    p = np.random.default_rng(5).permutation(cfg.E)
    ids2, wts2, *_ = oracle.route(x, W[p], b[p], 4)
    assert np.array_equal(p[ids2], ids)
    assert np.array_equal(wts2, wts)


def test_gap_flags():
    bias = np.array([0.3, 0.1, 0.2, 0.2 - 2e-5, -0.1], dtype=np.float32)
    ids, wts, lg, sg, gk, gi = _route_by_bias(bias, 3)
    c = (np.float32(0.5) + bias).astype(np.float64)
    assert list(ids[0]) == [0, 2, 3]
    assert gk[0] == pytest.approx(c[3] - c[1])
    assert gi[0] == pytest.approx(c[2] - c[3])


# ---------------------------------------------------------------------------
# O4b: group-limited selection ([EDGE0] §七 sigmoid-group, rules ① and ②)
# ---------------------------------------------------------------------------

def _route_groups_by_bias(bias, K, n_group, topk_group):
    E = len(bias)
    x = np.zeros((1, 8), dtype=np.float32)
    W = np.zeros((E, 8), dtype=np.float32)
    return oracle.route_groups(x, W, np.asarray(bias, dtype=np.float32), K, n_group, topk_group)


def _groups_brute_force(c, K, n_group, topk_group):
    """The definition by sorting: group score = fp32 sum of the group's two
    largest scores; keep the topk_group best groups (ties: lower group);
    top-K of the kept experts (ties: lower id)."""
    E = len(c)
    gsz = E // n_group
    score = []
    for g in range(n_group):
        top = sorted((np.float32(v) for v in c[g * gsz:(g + 1) * gsz]), reverse=True)
        score.append(np.float32(top[0]) + np.float32(top[1]) if gsz >= 2 else np.float32(top[0]))
    kept = sorted(range(n_group), key=lambda g: (-float(score[g]), g))[:topk_group]
    alive = [e for e in range(E) if e // gsz in kept]
    return sorted(alive, key=lambda e: (-float(c[e]), e))[:K], score, kept


def test_groups_equal_brute_force_sort_with_ties():
    rng = np.random.default_rng(21)
    for trial in range(400):
        n_group = int(rng.integers(1, 7))
        gsz = int(rng.integers(2, 5))
        E = n_group * gsz
        topk_group = int(rng.integers(1, n_group + 1))
        K = int(rng.integers(1, topk_group * gsz + 1))
        bias = rng.integers(-3, 4, size=E).astype(np.float32) / 4   # many ties
        ids, wts, logits, sig, gk, gi, gg = _route_groups_by_bias(bias, K, n_group, topk_group)
        c = (np.float32(0.5) + bias).astype(np.float32)
        want, _, _ = _groups_brute_force(c, K, n_group, topk_group)
        assert list(ids[0]) == want, (n_group, gsz, topk_group, K, bias)
        assert np.allclose(wts[0], 2.5 / K, rtol=0, atol=1e-6)


def test_groups_exclude_the_best_single_expert():
    # expert 0 has the best score, but its group's second is the worst: group
    # 0 scores 0.9 + (-0.9) and loses to groups 1 and 2
    bias = np.array([0.9, -0.9, 0.5, 0.4, 0.3, 0.3, 0.0, 0.0], dtype=np.float32) - 0.5
    ids, *_ = _route_groups_by_bias(bias, 2, 4, 2)
    assert list(ids[0]) == [2, 3]
    ids1, *_ = _route_by_bias(bias, 2)      # without groups expert 0 wins
    assert list(ids1[0]) == [0, 2]


def test_group_ties_keep_the_lower_group():
    # all four groups score 1.0: groups 0 and 1 are kept
    bias = np.array([0.1, -0.1, 0.2, -0.2, 0.0, 0.0, 0.3, -0.3], dtype=np.float32)
    ids, wts, lg, sg, gk, gi, gg = _route_groups_by_bias(bias, 4, 4, 2)
    assert sorted(ids[0].tolist()) == [0, 1, 2, 3]
    assert list(ids[0]) == [2, 0, 1, 3]
    assert gg[0] == 0.0


def test_all_groups_kept_is_plain_topk():
    cfg = synth.CONFIGS["tiny"]
    W = synth.router_weight(cfg, 0)
    b = synth.router_bias(cfg, 0)
    x = synth.tokens(cfg, T=12)
    ids, wts, lg, sg, gk, gi = oracle.route(x, W, b, 4)
    for ng in (2, 4, 8):
        ids2, wts2, lg2, sg2, gk2, gi2, gg2 = oracle.route_groups(x, W, b, 4, ng, ng)
        assert np.array_equal(ids2, ids) and np.array_equal(wts2, wts)
        assert np.all(np.isinf(gg2))


def test_groups_on_router_scores():
    """Real router scores: the selection is the sorting definition applied to
    c = sigma + bias, the weights renormalise the chosen sigmas, and gap_g is
    the kept/excluded group-score gap."""
    cfg = synth.CONFIGS["tiny"]
    W = synth.router_weight(cfg, 0)
    b = synth.router_bias(cfg, 0)
    x = synth.tokens(cfg, T=16, stream=3)
    ng, kg, K = 8, 3, 6
    ids, wts, lg, sg, gk, gi, gg = oracle.route_groups(x, W, b, K, ng, kg)
    for t in range(16):
        c = (sg[t] + b).astype(np.float32)
        want, score, kept = _groups_brute_force(c, K, ng, kg)
        assert list(ids[t]) == want
        s = sg[t, ids[t]].astype(np.float64)
        assert np.allclose(wts[t], 2.5 * s / s.sum(), rtol=1e-7)
        out = [g for g in range(ng) if g not in kept]
        assert gg[t] == pytest.approx(float(score[kept[-1]]) - max(float(score[g]) for g in out))


def test_groups_reject_bad_shapes():
    x = np.zeros((1, 8), dtype=np.float32)
    W = np.zeros((8, 8), dtype=np.float32)
    b = np.zeros(8, dtype=np.float32)
    for ng, kg, K in ((3, 1, 1), (8, 1, 1), (4, 5, 1), (4, 1, 3)):
        with pytest.raises(ValueError):
            oracle.route_groups(x, W, b, K, ng, kg)


# ---------------------------------------------------------------------------
# O4c: softmax scoring ([EDGE0] §七 softmax-top-k; [GLM-C] §05 olmoe step)
# ---------------------------------------------------------------------------

SM = oracle.SCORE_SOFTMAX


def test_softmax_equal_logits_uniform_and_lowest_ids():
    E, K = 16, 4
    x = np.zeros((1, 8), dtype=np.float32)
    W = np.zeros((E, 8), dtype=np.float32)
    b = np.linspace(-1, 1, E).astype(np.float32)          # ignored by softmax scoring
    ids, wts, lg, p, gk, gi = oracle.route(x, W, b, K, 1.0, 1, scoring=SM)
    assert np.all(p == np.float32(1.0 / E))
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.allclose(wts[0], 1.0 / K, rtol=0, atol=1e-7)       # renormalised to one
    ids, wts, *_ = oracle.route(x, W, b, K, 1.0, 0, scoring=SM)
    assert np.allclose(wts[0], 1.0 / E, rtol=0, atol=1e-8)       # raw probabilities
    assert gk[0] == 0.0


def test_softmax_matches_numpy_and_sorting_definition():
    cfg = synth.CONFIGS["tiny"]
    W = synth.router_weight(cfg, 0)
    b = synth.router_bias(cfg, 0)
    x = synth.tokens(cfg, T=16, stream=9)
    K = 4
    ids, wts, lg, p, gk, gi = oracle.route(x, W, b, K, 1.0, 1, scoring=SM)
    ref = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    ref /= ref.sum(axis=1, keepdims=True)
    assert np.allclose(p, ref, rtol=2e-7, atol=0)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-6)
    for t in range(16):
        want = sorted(range(cfg.E), key=lambda e: (-float(p[t, e]), e))[:K]
        assert list(ids[t]) == want
        s = p[t, ids[t]].astype(np.float64)
        assert np.allclose(wts[t], s / s.sum(), rtol=1e-7)
        lgs = sorted(lg[t].tolist(), reverse=True)
        assert gk[t] == pytest.approx(lgs[K - 1] - lgs[K])          # logit units
    ids0, wts0, *_ = oracle.route(x, W, b, K, 2.0, 0, scoring=SM)
    assert np.array_equal(ids0, ids)
    for t in range(16):
        assert np.allclose(wts0[t], 2.0 * p[t, ids[t]], rtol=1e-7)


def test_softmax_shift_invariance_and_bias_ignored():
    cfg = synth.CONFIGS["tiny"]
    W = synth.router_weight(cfg, 0)
    x = synth.tokens(cfg, T=8, stream=4)
    # a constant input column with equal weights shifts every logit equally
    x1 = np.concatenate([x, np.ones((8, 1), np.float32)], axis=1)
    W1 = np.concatenate([W, np.full((cfg.E, 1), 3.0, np.float32)], axis=1)
    W0 = np.concatenate([W, np.zeros((cfg.E, 1), np.float32)], axis=1)
    z = np.zeros(cfg.E, np.float32)
    ids_a, wts_a, _, p_a, *_ = oracle.route(x1, W0, z, 4, 1.0, 1, scoring=SM)
    ids_b, wts_b, _, p_b, *_ = oracle.route(x1, W1, z + 5.0, 4, 1.0, 1, scoring=SM)
    assert np.array_equal(ids_a, ids_b)
    assert np.allclose(p_a, p_b, rtol=2e-6, atol=0)
    assert np.allclose(wts_a, wts_b, rtol=2e-6)


def test_softmax_with_groups_is_rejected():
    x = np.zeros((1, 8), dtype=np.float32)
    W = np.zeros((8, 8), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.route_groups(x, W, np.zeros(8, np.float32), 2, 2, 1, scoring=SM)


# ---------------------------------------------------------------------------
# O5: bucketing
# ---------------------------------------------------------------------------

def test_bucket_brute_force_and_invariants():
    rng = np.random.default_rng(2)
    for trial in range(100):
        E = int(rng.integers(1, 20))
        K = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 12))
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        cnt, off, perm, active = oracle.bucket(ids, E)
        flat = ids.reshape(-1)
        assert cnt.sum() == T * K
        assert np.array_equal(np.sort(perm), np.arange(T * K))
        want = sorted(range(T * K), key=lambda a: (flat[a], a))
        assert list(perm) == want
        assert list(active) == sorted(set(flat.tolist()))
        assert len(active) <= min(T * K, E)
        for e in range(E):
            seg = perm[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------------------
# O6 / O7: expert math and combine, closed forms
# ---------------------------------------------------------------------------

def _row_blob(H, I, qg, qu, qd, sg, su, sd):
    """Builds a row-format blob from integer codes directly (no quantiser)."""
    def pack(qm):
        qm = np.asarray(qm, dtype=np.int64)
        n = qm & 0xF
        return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)
    parts = [pack(qg).ravel(), pack(qu).ravel(), pack(qd).ravel(),
             np.asarray(sg, np.float32).view(np.uint8), np.asarray(su, np.float32).view(np.uint8),
             np.asarray(sd, np.float32).view(np.uint8)]
    blob = np.concatenate(parts)
    assert blob.size == oracle.blob_bytes(ROW, H, I)
    return blob


def test_expert_all_ones_closed_form():
    H, I = 64, 32
    ones = np.ones
    blob = _row_blob(H, I, ones((I, H)), ones((I, H)), ones((H, I)), ones(I), ones(I), ones(H))
    x = np.full(H, 1 / 8, dtype=np.float32)        # sum(x) = 8
    y, h = oracle.expert(ROW, H, I, blob, x)
    h_want = 8.0 / (1 + math.exp(-8.0)) * 8.0
    assert np.allclose(h, h_want, rtol=1e-7)
    assert np.allclose(y, I * np.float32(h_want), rtol=1e-7)


def test_expert_single_weight_closed_form():
    H, I = 64, 32
    qg = np.zeros((I, H)); qu = np.zeros((I, H)); qd = np.zeros((H, I))
    qg[5, 9] = 3
    qu[5, 20] = -2
    qd[:, 5] = np.arange(H) % 15 - 7
    sg = np.full(I, 0.5); su = np.full(I, 0.25); sd = np.linspace(0.1, 1.0, H)
    blob = _row_blob(H, I, qg, qu, qd, sg, su, sd)
    x = synth.gauss(synth.key(1, 0, synth.T_X, 9), H, 1.0)
    y, h = oracle.expert(ROW, H, I, blob, x)
    g = np.float32(1.5 * float(x[9]))
    u = np.float32(-0.5 * float(x[20]))
    hw = np.float32(float(g) / (1 + math.exp(-float(g))) * float(u))
    assert h[5] == pytest.approx(float(hw), rel=1e-7)
    assert np.all(np.delete(h, 5) == 0)
    want = sd.astype(np.float32).astype(np.float64) * qd[:, 5] * float(hw)
    assert np.allclose(y, want, rtol=1e-6)


def test_expert_zero_weights_give_zero():
    H, I = 64, 64
    z = np.zeros
    blob = _row_blob(H, I, z((I, H)), z((I, H)), z((H, I)), np.ones(I), np.ones(I), np.ones(H))
    y, h = oracle.expert(ROW, H, I, blob, synth.tokens(synth.CONFIGS["tiny"])[0, :64])
    assert not y.any() and not h.any()


def test_affine_expert_constant_groups_closed_form():
    H, I = 128, 64
    wg = np.full((I, H), 0.125, dtype=np.float32)
    wu = np.full((I, H), -0.0625, dtype=np.float32)
    wd = np.full((H, I), 0.5, dtype=np.float32)
    blob = oracle.pack_expert(AFF, wg, wu, wd)
    x = np.linspace(-1, 1, H).astype(np.float32) + 0.25
    sx = float(x.astype(np.float64).sum())
    y, h = oracle.expert(AFF, H, I, blob, x)
    g, u = np.float32(0.125 * sx), np.float32(-0.0625 * sx)
    hw = np.float32(float(g) / (1 + math.exp(-float(g))) * float(u))
    assert np.allclose(h, hw, rtol=1e-7)
    assert np.allclose(y, 0.5 * I * float(hw), rtol=1e-6)


@pytest.mark.parametrize("fmt", [ROW, AFF])
def test_blob_layout_round_trips_exact_weights(fmt):
    H, I = 128, 64
    rng = np.random.default_rng(4)
    if fmt == ROW:
        def mk(O, In):
            q = rng.integers(-7, 8, size=(O, In)); q[:, 0] = 7
            return (q * 2.0 ** -7).astype(np.float32)
    else:
        def mk(O, In):
            q = rng.integers(0, 16, size=(O, In)); q[:, ::64] = 0; q[:, 1::64] = 15
            return (q * 2.0 ** -7 - 0.0625).astype(np.float32)
    wg, wu, wd = mk(I, H), mk(I, H), mk(H, I)
    blob = oracle.pack_expert(fmt, wg, wu, wd)
    dg, du, dd = oracle.dequant_expert(fmt, H, I, blob)
    assert np.array_equal(dg, wg) and np.array_equal(du, wu) and np.array_equal(dd, wd)


def test_combine_closed_forms():
    T, K, H = 2, 3, 5
    yr = np.arange(T * K * H, dtype=np.float32).reshape(T * K, H)
    w = np.array([[2.5, 0, 0], [0, 0, 2.5]], dtype=np.float32)
    ys = np.ones((1, T, H), dtype=np.float32)
    out = oracle.combine(yr, w, ys, 1)
    assert np.array_equal(out[0], 2.5 * yr[0] + 1)
    assert np.array_equal(out[1], 2.5 * yr[5] + 1)


# ---------------------------------------------------------------------------
# whole layer: invariants that pin composition
# ---------------------------------------------------------------------------

def _tiny_layer(cfg, n_tok=None):
    W = synth.router_weight(cfg, 0)
    b = synth.router_bias(cfg, 0)
    blobs = [oracle.pack_expert(cfg.fmt, *synth.expert_weights(cfg, 0, e)) for e in range(cfg.E)]
    shared = [oracle.pack_expert(cfg.fmt, *synth.expert_weights(cfg, 0, cfg.E + s))
              for s in range(cfg.n_shared)]
    x = synth.tokens(cfg, T=n_tok)
    return W, b, blobs, shared, x


def test_layer_identical_experts_sum_to_routed_scale():
    cfg = synth.CONFIGS["tiny"]
    W, b, blobs, shared, x = _tiny_layer(cfg)
    same = [blobs[0]] * cfg.E
    out, ids, wts = oracle.moe_layer(x, W, b, cfg.K, cfg.fmt, cfg.I, same, shared)
    for t in range(cfg.T):
        y, _ = oracle.expert(cfg.fmt, cfg.H, cfg.I, blobs[0], x[t])
        ysh, _ = oracle.expert(cfg.fmt, cfg.H, cfg.I, shared[0], x[t])
        assert np.allclose(out[t], 2.5 * y.astype(np.float64) + ysh, rtol=1e-6, atol=1e-6)


def test_layer_relabelling_and_token_independence():
    cfg = synth.CONFIGS["tiny"]
    W, b, blobs, shared, x = _tiny_layer(cfg)
    out, ids, wts = oracle.moe_layer(x, W, b, cfg.K, cfg.fmt, cfg.I, blobs, shared)
    p = np.random.default_rng(8).permutation(cfg.E)
    out2, ids2, _ = oracle.moe_layer(x, W[p], b[p], cfg.K, cfg.fmt, cfg.I,
                                     [blobs[e] for e in p], shared)
    assert np.array_equal(out, out2) and np.array_equal(p[ids2], ids)
    for t in range(cfg.T):
        o1, _, _ = oracle.moe_layer(x[t:t + 1], W, b, cfg.K, cfg.fmt, cfg.I, blobs, shared)
        assert np.array_equal(o1[0], out[t])


def test_layer_missing_expert_is_an_error():
    cfg = synth.CONFIGS["tiny"]
    W, b, blobs, shared, x = _tiny_layer(cfg)
    _, ids, _ = oracle.moe_layer(x, W, b, cfg.K, cfg.fmt, cfg.I, blobs, shared)
    holes = list(blobs)
    holes[int(ids[0, 0])] = None
    with pytest.raises(ValueError):
        oracle.moe_layer(x, W, b, cfg.K, cfg.fmt, cfg.I, holes, shared)


def _ones_blob(H, I, s_gu=1.0, s_d=1.0):
    """Row-format blob with every code +1: gate/up row scales s_gu, down s_d."""
    blob = np.full(oracle.blob_bytes(ROW, H, I), 0x11, dtype=np.uint8)
    sc = np.concatenate([np.full(2 * I, s_gu), np.full(H, s_d)]).astype(np.float32)
    blob[3 * H * I // 2:] = sc.view(np.uint8)
    return blob


def test_residual_layer_closed_form():
    """x <- x + moe(rmsnorm(x)) with a routed expert and a shared expert whose
    codes are all +1: for v = rmsnorm(x) and S = sum(v), an all-ones gate/up
    row with scale s gives g = u = s*S, h = silu(s*S) * s*S, and the all-ones
    down rows give y = I*h; the one chosen expert (K = 1, renormalised weight
    = routed_scale) enters with 2.5, the shared expert with 1.  Written in
    float64 from x directly: S = sum(x) / sqrt(mean(x^2) + eps)."""
    H, I, E, eps = 64, 32, 4, 1e-6
    x = (synth.gauss(synth.key(31, 0, synth.T_X, 0), 3 * H, 1.0) * 3.0).reshape(3, H)
    W = np.zeros((E, H), np.float32)
    b = np.array([0.0, 0.3, 0.0, 0.1], np.float32)       # sigma = 0.5 everywhere: expert 1 wins
    zero = np.zeros(oracle.blob_bytes(ROW, H, I), np.uint8)
    blobs = [zero, _ones_blob(H, I), zero, zero]
    shared = [_ones_blob(H, I, s_gu=0.5)]
    got, ids, wts = oracle.residual_layer(x, W, b, 1, ROW, I, blobs, shared, eps=eps)
    assert np.all(ids == 1) and np.all(wts == np.float32(2.5))
    xd = x.astype(np.float64)
    S = xd.sum(axis=1) / np.sqrt((xd * xd).mean(axis=1) + eps)
    silu = lambda z: z / (1 + np.exp(-z))
    term = 2.5 * I * S * silu(S) + I * (0.5 * S) * silu(0.5 * S)
    want = xd + term[:, None]
    assert np.allclose(got, want, rtol=2e-6, atol=2e-6 * np.abs(term).max())
    # the other readings differ: no norm (x + moe(x)) or the norm after the add
    S_raw = xd.sum(axis=1)
    assert not np.allclose(got[:, 0], xd[:, 0] + 2.5 * I * S_raw * silu(S_raw), rtol=1e-3)
    # zero experts: x comes back bit for bit
    same, _, _ = oracle.residual_layer(x, W, b, 1, ROW, I, [zero] * E, [zero], eps=eps)
    assert np.array_equal(same, x)


def test_rmsnorm_closed_form_and_scale_invariance():
    x = np.full((1, 64), -3.0, dtype=np.float32)
    out = oracle.rmsnorm(x, eps=0.0)
    assert np.all(out == -1.0)
    y = synth.tokens(synth.CONFIGS["tiny"])
    a = oracle.rmsnorm(y, eps=0.0)
    b = oracle.rmsnorm(8 * y, eps=0.0)
    assert np.array_equal(a, b)
    assert np.allclose((a.astype(np.float64) ** 2).mean(axis=1), 1.0, rtol=1e-6)


# ---------------------------------------------------------------------------
# O0: the converter step before the path ([GLM-C] §06): FP8 E4M3 with block
# inverse scales, bf16, and the offset-binary container
# ---------------------------------------------------------------------------

def _f8(values):
    """fp32 values exactly representable in E4M3 -> their codes (torch's encoder)."""
    torch = pytest.importorskip("torch")
    return torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_fp8_decode_matches_torch_on_every_code():
    torch = pytest.importorskip("torch")
    c = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_e4m3_to_f32(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert list(np.where(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_fp8_decode_closed_forms():
    d = lambda b: float(oracle.fp8_e4m3_to_f32([b])[0])  # noqa: E731
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0xB8) == -1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert d(0x08) == 2.0 ** -6                             # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9  # subnormals
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert d(0x3C) == 1.5 and d(0x44) == 3.0


def test_fp8_block_dequant_matches_page_expression():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    O, I = 300, 200                                   # ragged in both block dims
    q = rng.integers(0, 256, size=(O, I), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x33                      # no NaN codes
    sinv = rng.uniform(1e-5, 1e-2, size=(3, 2)).astype(np.float32)
    got = oracle.dequant_fp8_block(q, sinv)
    w = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    sc = torch.from_numpy(sinv).repeat_interleave(128, 0).repeat_interleave(128, 1)[:O, :I]
    assert np.array_equal(got.view(np.uint32), (w * sc).numpy().view(np.uint32))


def test_fp8_block_boundaries():
    O, I = 260, 390
    q = np.full((O, I), 0x38, dtype=np.uint8)        # every code 1.0
    sinv = np.array([[2.0 ** (4 * a + b) for b in range(4)] for a in range(3)], dtype=np.float32)
    w = oracle.dequant_fp8_block(q, sinv)
    oo, ii = np.meshgrid(np.arange(O), np.arange(I), indexing="ij")
    assert np.array_equal(w, sinv[oo // 128, ii // 128])


def test_bf16_decode():
    torch = pytest.importorskip("torch")
    b = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3E4C], dtype=np.uint16)
    w = oracle.bf16_to_f32(b)
    assert list(w[:5]) == [1.0, -2.0, 0.0, -0.0, np.inf] and math.copysign(1, w[3]) == -1
    r = np.random.default_rng(3).integers(0, 0x7F80, size=1000).astype(np.uint16)
    ref = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_to_f32(r).view(np.uint32), ref.view(np.uint32))


def test_requant_fp8_on_the_grid_gives_the_integers():
    rng = np.random.default_rng(5)
    O, I = 130, 256
    ints = rng.integers(-7, 8, size=(O, I))
    ints[:, 7] = 7                                    # row max 7: s = sinv exactly
    q = _f8(ints)
    # one power of two per row block, the same for both column blocks
    sinv = np.repeat(2.0 ** rng.integers(-12, -4, size=(2, 1)), 2, axis=1).astype(np.float32)
    codes, s = oracle.requant_int4_rows(q, oracle.SRC_FP8_E4M3, sinv)
    assert np.array_equal(s, sinv[np.arange(O) // 128, 0])
    assert np.array_equal(oracle.unpack_int4_row(codes, I).astype(int), ints)


def test_requant_ties_go_to_even():
    # row max 7 with sinv 1: s = 1, so w / s is w itself; halves round to even
    vals = [7.0, 2.5, 3.5, -2.5, 1.5, -0.5, 0.5, -1.5, 5.5, -6.5, 4.5, 0.0]
    want = [7, 2, 4, -2, 2, 0, 0, -2, 6, -6, 4, 0]
    q = _f8([vals])
    codes, s = oracle.requant_int4_rows(q, oracle.SRC_FP8_E4M3, np.ones((1, 1), np.float32))
    assert s[0] == 1.0
    assert list(oracle.unpack_int4_row(codes, len(vals))[0]) == want


def test_requant_bf16_equals_pack_of_widened_values():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)
    b = (w.view(np.uint32) >> 16).astype(np.uint16)   # truncated to bf16 bits
    widened = (b.astype(np.uint32) << 16).view(np.float32)
    codes, s = oracle.requant_int4_rows(b, oracle.SRC_BF16)
    c2, s2 = oracle.pack_int4_row(widened)
    assert np.array_equal(codes, c2) and np.array_equal(s, s2)


def test_container_converter_is_the_blob_with_flipped_nibbles():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0                                        # floor row
    qc, sc = oracle.convert_int4_container(w)
    qb, sb = oracle.pack_int4_row(w)
    assert np.array_equal(sc, sb)
    assert np.array_equal(qc, qb ^ 0x88)


def test_container_converter_reproduces_page_bytes():
    g = _golden("int4_container_example.txt")
    raw = [int(b, 16) for b in g["bytes_offset_binary"].split()]
    codes = []
    for b in raw:
        codes += [(b & 0xF) - 8, (b >> 4) - 8]
    row = np.array(codes + [7, 0], dtype=np.float32) * 0.25   # a 7 fixes s = 0.25
    q, s = oracle.convert_int4_container(row[None, :])
    assert s[0] == 0.25
    assert list(q[0, :8]) == raw


# ---------------------------------------------------------------------------
# O1b: per-row int8 ([GLM-C] §05 quantize_rows, bits = 8), the shared
# expert's format option
# ---------------------------------------------------------------------------

I8 = oracle.W_INT8_ROW


def test_int8_blob_is_one_byte_per_weight():
    # the page's int8 expert slot: one byte per parameter plus one fp32 scale per row
    for H, I in [(6144, 2048), (512, 256)]:
        assert oracle.blob_bytes(I8, H, I) == 3 * H * I + 4 * (2 * I + H)


def test_int8_on_grid_values_come_back_exactly():
    rng = np.random.default_rng(21)
    k = rng.integers(-127, 128, size=(40, 96))
    k[:, 3] = 127                                        # row max 127: s = step exactly
    step = (2.0 ** rng.integers(-12, -4, size=(40, 1))).astype(np.float32)
    q, s = oracle.pack_int8_row((k * step).astype(np.float32))
    assert np.array_equal(s, step[:, 0])
    assert np.array_equal(q.astype(int), k)


def test_int8_ties_floor_and_bound():
    w = np.array([[127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 126.5, -126.5]], dtype=np.float32)
    q, s = oracle.pack_int8_row(w)
    assert s[0] == 1.0 and list(q[0]) == [127, 2, 4, -2, 0, 0, 126, -126]
    q, s = oracle.pack_int8_row(np.zeros((2, 64), np.float32))
    assert np.all(s == np.float32(1e-8)) and np.all(q == 0)
    w = (np.random.default_rng(2).standard_normal((64, 256)) * 0.02).astype(np.float32)
    q, s = oracle.pack_int8_row(w)
    assert q.min() >= -127 and q.max() <= 127            # s = amax/127: -128 never occurs
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * 0.5 * (1 + 1e-6))


def test_int8_expert_closed_form():
    # constant weights c: codes are all 127, dequantised exactly to c
    H, I, c = 128, 64, 0.015625
    x = np.random.default_rng(3).standard_normal(H).astype(np.float32)
    blob = oracle.pack_expert(I8, np.full((I, H), c, np.float32), np.full((I, H), c, np.float32),
                              np.full((H, I), c, np.float32))
    y, h = oracle.expert(I8, H, I, blob, x)
    g = c * x.astype(np.float64).sum()
    hv = np.float32(g / (1 + np.exp(-g)) * g)
    assert np.allclose(h, hv, rtol=1e-6)
    assert np.allclose(y, c * I * np.float64(hv), rtol=1e-6)


def test_layer_with_int8_shared_is_routed_plus_shared():
    rng = np.random.default_rng(4)
    H, I, E, K = 128, 64, 8, 2
    x = rng.standard_normal((3, H)).astype(np.float32)
    Wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    mk = lambda fmt: oracle.pack_expert(fmt, *(  # noqa: E731
        (rng.standard_normal(sh) * 0.02).astype(np.float32) for sh in [(I, H), (I, H), (H, I)]))
    blobs = [mk(ROW) for _ in range(E)]
    sh = mk(I8)
    out, ids, wts = oracle.moe_layer(x, Wr, b, K, ROW, I, blobs, [sh], shared_fmt=I8)
    for t in range(3):
        ref = oracle.expert(I8, H, I, sh, x[t])[0].astype(np.float64)
        for k in range(K):
            ref += wts[t, k] * oracle.expert(ROW, H, I, blobs[ids[t, k]], x[t])[0]
        assert np.allclose(out[t], ref, rtol=1e-5, atol=1e-7)
