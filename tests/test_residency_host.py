"""Host-side residency logic of the library, no GPU: the staged executor's
slot choice (sticky slots, Edge0 write-up §十四) and the slot image an
asynchronous load copies.  Both are plain host functions of the C ABI."""
import numpy as np
import pytest

from int4_weight_expert_amd import moe as M

ROW, AFF = M.MOE_W_INT4_ROW, M.MOE_W_INT4_AFFINE_G64


def ref_plan(held, used, want):
    """The rule written out: keep held wanted experts; fill empty slots in
    ascending order, then the least recently wanted (ties: lower slot)."""
    slot_of, load = [None] * len(want), [0] * len(want)
    taken = set()
    for i, w in enumerate(want):
        if w in held:
            j = held.index(w)
            slot_of[i] = j
            taken.add(j)
    free = [j for j in range(len(held)) if j not in taken]
    free.sort(key=lambda j: (held[j] >= 0, used[j], j))
    k = 0
    for i in range(len(want)):
        if slot_of[i] is None:
            slot_of[i], load[i] = free[k], 1
            k += 1
    return k, slot_of, load


def test_sticky_plan_cases():
    n, so, ld = M.moe_sticky_plan([3, 5, 7, -1], [0, 0, 0, -1], [5, 3])
    assert n == 0 and list(so) == [1, 0] and list(ld) == [0, 0]
    n, so, ld = M.moe_sticky_plan([-1, 4, -1, 9], [-1, 5, -1, 2], [4, 1, 2])
    assert n == 2 and list(so) == [1, 0, 2] and list(ld) == [0, 1, 1]
    n, so, ld = M.moe_sticky_plan([1, 2, 3, 4], [5, 1, 3, 2], [9, 8])
    assert n == 2 and list(so) == [1, 3] and list(ld) == [1, 1]


def test_sticky_plan_rejects():
    assert M.moe_sticky_plan([1, 2], [0, 0], [1, 2, 3])[0] == -1      # more wanted than slots
    assert M.moe_sticky_plan([1, 2, 3], [0, 0, 0], [4, 4])[0] == -1   # repeated id
    assert M.moe_sticky_plan([1, 2, 3], [0, 0, 0], [-2])[0] == -1     # negative id


def test_sticky_plan_matches_rule_on_random_steps():
    rng = np.random.default_rng(17)
    for trial in range(300):
        P = int(rng.integers(1, 12))
        E = int(rng.integers(P, 40))
        held = [-1] * P
        used = [-1] * P
        for step in range(6):
            n = int(rng.integers(0, P + 1))
            want = [int(v) for v in rng.choice(E, size=n, replace=False)]
            n_ld, so, ld = M.moe_sticky_plan(held, used, want)
            r_n, r_so, r_ld = ref_plan(held, used, want)
            assert n_ld == r_n and list(so) == r_so and list(ld) == r_ld
            assert len(set(so.tolist())) == n
            assert n_ld == len(set(want) - set(held))
            for i, w in enumerate(want):
                held[so[i]] = w
                used[so[i]] = step


def ref_image(fmt, H, I, blob):
    """The slot order as documented: matrix [O][In/2] in 8-row groups, group
    q chunk c (16 bytes, 32 inputs) of row 8q+r at ((q*In/32+c)*8+r)*16,
    row-format codes offset binary (byte ^ 0x88); row scales as they are;
    affine (scale, min) pairs of (row, group) at ((q*In/64+g)*8+r)*4."""
    out = np.empty_like(blob)
    gq, dq = I * H // 2, H * I // 2
    flip = 0x88 if fmt == ROW else 0
    for off, O, In in [(0, I, H), (gq, I, H), (2 * gq, H, I)]:
        m = blob[off:off + O * In // 2].reshape(O // 8, 8, In // 32, 16)
        out[off:off + O * In // 2] = (m.transpose(0, 2, 1, 3) ^ flip).reshape(-1)
    sb = 2 * gq + dq
    if fmt == ROW:
        out[sb:] = blob[sb:]
    else:
        ga = I * (H // 64) * 4
        for off, O, G in [(sb, I, H // 64), (sb + ga, I, H // 64), (sb + 2 * ga, H, I // 64)]:
            m = blob[off:off + O * G * 4].reshape(O // 8, 8, G, 4)
            out[off:off + O * G * 4] = m.transpose(0, 2, 1, 3).reshape(-1)
    return out


@pytest.mark.parametrize("fmt,H,I", [(ROW, 128, 64), (ROW, 512, 256), (AFF, 128, 128),
                                     (AFF, 256, 512)])
def test_blob_to_image_matches_documented_layout(fmt, H, I):
    nb = M.lib().moe_image_bytes(fmt, H, I)
    blob = np.random.default_rng(H + I).integers(0, 256, size=nb, dtype=np.uint8)
    img = M.moe_blob_to_image(fmt, H, I, blob)
    assert np.array_equal(img, ref_image(fmt, H, I, blob))


def test_blob_to_image_rejects():
    blob = np.zeros(M.lib().moe_image_bytes(ROW, 128, 64), dtype=np.uint8)
    out = np.empty_like(blob)
    L = M.lib()
    assert L.moe_blob_to_image(ROW, 128, 64, blob.ctypes.data, blob.nbytes - 1,
                               out.ctypes.data) == M.MOE_E_SIZE
    assert L.moe_blob_to_image(ROW, 100, 64, blob.ctypes.data, blob.nbytes,
                               out.ctypes.data) == M.MOE_E_ARG
    assert L.moe_blob_to_image(5, 128, 64, blob.ctypes.data, blob.nbytes,
                               out.ctypes.data) == M.MOE_E_ARG
    assert L.moe_image_bytes(ROW, 6144, 2048) == 18915328
    assert L.moe_image_bytes(AFF, 2048, 512) == 1769472
