"""An independent float64 recomputation of the tiny layer (H=512, E=32,
top-4, I=256, one shared expert, T=4, seed 0) from the same packed bytes,
written here in NumPy without any oracle routine: the nibbles are decoded,
the router, the SwiGLU experts and the weighted combine are evaluated in
float64 with no intermediate rounding.  The oracle rounds each named
intermediate to fp32, so the two agree to a few fp32 ulps; the ids must be
identical.

Sources of what is computed: the GLM-5.2 engine page ("惊呆了！25GB 内存上运
行 GLM 5.2 744B 模型", reader.mx) §11 (sigmoid plus correction bias picks,
the plain sigmoid weighs; SwiGLU on the gathered rows), §06 (per-row int4
codes, two per byte, first column in the low nibble); the GLM-5.2 dataflow
page (devpress) §三 Step 6c-6d (the shared expert added with weight 1); the
Edge0 write-up §七 (weights renormalised with a 1e-20 term)."""
import numpy as np

import oracle
import synth

CFG = synth.CONFIGS["tiny"]


def _decode_row_blob(blob, H, I):
    """(Wg [I][H], Wu [I][H], Wd [H][I]) in float64 from a row-format blob:
    two's-complement nibbles, low nibble first, then fp32 row scales."""
    def mat(raw, O, In):
        b = raw.reshape(O, In // 2).astype(np.int64)
        lo, hi = b & 0xF, b >> 4
        q = np.empty((O, In), np.int64)
        q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
        q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
        return q.astype(np.float64)
    gq = I * H // 2
    qg = mat(blob[:gq], I, H)
    qu = mat(blob[gq:2 * gq], I, H)
    qd = mat(blob[2 * gq:3 * gq], H, I)
    sc = blob[3 * gq:].view(np.float32).astype(np.float64)
    sg, su, sd = sc[:I], sc[I:2 * I], sc[2 * I:]
    return qg * sg[:, None], qu * su[:, None], qd * sd[:, None]


def _expert(w, x):
    wg, wu, wd = w
    g, u = wg @ x, wu @ x
    h = g / (1.0 + np.exp(-g)) * u
    return wd @ h


def test_tiny_layer_float64_recomputation():
    H, I, E, K = CFG.H, CFG.I, CFG.E, CFG.K
    W = synth.router_weight(CFG, 0).astype(np.float64)
    b = synth.router_bias(CFG, 0).astype(np.float64)
    blobs = [oracle.pack_expert(CFG.fmt, *synth.expert_weights(CFG, 0, e)) for e in range(E)]
    shared = oracle.pack_expert(CFG.fmt, *synth.expert_weights(CFG, 0, E))
    x = synth.tokens(CFG)
    got, ids, wts = oracle.moe_layer(x, synth.router_weight(CFG, 0), synth.router_bias(CFG, 0),
                                     K, CFG.fmt, I, blobs, [shared])

    dec = [_decode_row_blob(bl, H, I) for bl in blobs]
    dsh = _decode_row_blob(shared, H, I)
    for t in range(CFG.T):
        xt = x[t].astype(np.float64)
        sig = 1.0 / (1.0 + np.exp(-(W @ xt)))
        score = sig + b
        order = sorted(range(E), key=lambda e: (-score[e], e))
        top = order[:K]
        assert score[order[K - 1]] - score[order[K]] > 1e-4   # no near tie on this seed
        assert list(ids[t]) == top
        w = 2.5 * sig[top] / (sig[top].sum() + 1e-20)
        assert np.allclose(wts[t], w, rtol=1e-6)
        want = _expert(dsh, xt) + sum(w[k] * _expert(dec[top[k]], xt) for k in range(K))
        err = np.abs(got[t] - want).max() / np.abs(want).max()
        assert err < 1e-5, (t, err)
