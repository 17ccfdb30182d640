"""ctypes binding of the plain C CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports this package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(_HERE, "libmoe_oracle.so")
# a differently built copy of the same source (e.g. with sanitizers) may be
# loaded instead; build() still writes the default library
_LOAD = os.environ.get("MOE_ORACLE_SO", SO)

W_INT4_ROW = 1
W_INT4_AFFINE_G64 = 2
W_INT8_ROW = 3


def build() -> None:
    """Compile the oracle with gcc (single-threaded, IEEE fp, no fast-math)."""
    subprocess.check_call(
        ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
         os.path.join(_HERE, "moe_oracle.c"), "-o", SO + ".tmp", "-lm"])
    os.replace(SO + ".tmp", SO)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if _LOAD == SO and not os.path.exists(SO):
            build()
        L = ctypes.CDLL(_LOAD)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.orc_blob_bytes.argtypes = [i32, i64, i64]
        L.orc_blob_bytes.restype = i64
        L.orc_bf16_round.argtypes = [f32]
        L.orc_bf16_round.restype = f32
        L.orc_pack_int4_row.argtypes = [vp, i64, i64, vp, vp]
        L.orc_unpack_int4_row.argtypes = [vp, i64, i64, vp]
        L.orc_dequant_int4_row.argtypes = [vp, vp, i64, i64, vp]
        L.orc_pack_affine_g64.argtypes = [vp, i64, i64, vp, vp]
        L.orc_dequant_affine_g64.argtypes = [vp, vp, i64, i64, vp]
        L.orc_pack_expert.argtypes = [i32, i64, i64, vp, vp, vp, vp]
        L.orc_pack_expert.restype = i32
        L.orc_dequant_expert.argtypes = [i32, i64, i64, vp, vp, vp, vp]
        L.orc_dequant_expert.restype = i32
        L.orc_expert.argtypes = [i32, i64, i64, vp, vp, vp, vp]
        L.orc_expert.restype = i32
        L.orc_route.argtypes = [vp, i32, i64, vp, vp, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp]
        L.orc_route.restype = i32
        L.orc_route_full.argtypes = [vp, i32, i64, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp,
                                     vp, vp, vp, vp, vp, vp]
        L.orc_route_full.restype = i32
        L.orc_bucket.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_bucket.restype = i32
        L.orc_combine.argtypes = [i32, i32, i64, i32, vp, vp, vp, vp]
        L.orc_combine.restype = None
        L.orc_moe_layer.argtypes = [vp, i32, i64, i64, i32, i32, i32, vp, vp, f32, i32, vp, i32,
                                    vp, vp, vp, vp]
        L.orc_moe_layer.restype = i32
        L.orc_moe_layer_full.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, vp, vp, i32, i32, i32,
                                         f32, i32, vp, i32, vp, vp, vp, vp]
        L.orc_moe_layer_full.restype = i32
        L.orc_rmsnorm.argtypes = [vp, i32, i64, f32, vp]
        L.orc_rmsnorm.restype = None
        L.orc_residual_layer.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, vp, vp, i32, i32,
                                         i32, f32, i32, vp, i32, vp, f32, vp, vp]
        L.orc_residual_layer.restype = i32
        L.orc_fp8_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_fp8_e4m3_to_f32.restype = f32
        L.orc_dequant_fp8_block.argtypes = [vp, vp, i64, i64, i64, vp]
        L.orc_bf16_to_f32.argtypes = [vp, i64, vp]
        L.orc_convert_int4_container.argtypes = [vp, i64, i64, vp, vp]
        L.orc_pack_int8_row.argtypes = [vp, i64, i64, vp, vp]
        L.orc_pack_int8_row.restype = None
        for name in ("orc_dequant_fp8_block", "orc_bf16_to_f32", "orc_convert_int4_container"):
            getattr(L, name).restype = None
        for name in ("orc_pack_int4_row", "orc_unpack_int4_row", "orc_dequant_int4_row",
                     "orc_pack_affine_g64", "orc_dequant_affine_g64"):
            getattr(L, name).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def blob_bytes(fmt: int, H: int, I: int) -> int:
    return int(lib().orc_blob_bytes(fmt, H, I))


def bf16_round(v: float) -> float:
    return float(lib().orc_bf16_round(v))


def pack_int4_row(w: np.ndarray):
    w = _f32(w)
    O, I = w.shape
    q = np.empty((O, (I + 1) // 2), dtype=np.uint8)
    s = np.empty(O, dtype=np.float32)
    lib().orc_pack_int4_row(_p(w), O, I, _p(q), _p(s))
    return q, s


SRC_F32, SRC_BF16, SRC_FP8_E4M3 = 0, 1, 2
FP8_BLOCK = 128


def fp8_e4m3_to_f32(codes) -> np.ndarray:
    """FP8 E4M3 (fn) codes -> fp32, code by code ([GLM-C] §06)."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.array([lib().orc_fp8_e4m3_to_f32(int(v)) for v in c.reshape(-1)], dtype=np.float32)
    return out.reshape(c.shape)


def dequant_fp8_block(q: np.ndarray, sinv: np.ndarray, block: int = FP8_BLOCK) -> np.ndarray:
    """fp8 [O][I] times its [ceil(O/B)][ceil(I/B)] inverse block scales ([GLM-C] §06)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    O, I = q.shape
    sinv = _f32(sinv)
    assert sinv.shape == ((O + block - 1) // block, (I + block - 1) // block)
    w = np.empty((O, I), dtype=np.float32)
    lib().orc_dequant_fp8_block(_p(q), _p(sinv), O, I, block, _p(w))
    return w


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    w = np.empty(b.shape, dtype=np.float32)
    lib().orc_bf16_to_f32(_p(b), b.size, _p(w))
    return w


def decode_source(w, src: int, sinv=None) -> np.ndarray:
    """Checkpoint tensor -> fp32: fp32 as is, bf16 bits widened, FP8 E4M3
    codes times their block inverse scales ([GLM-C] §06)."""
    if src == SRC_F32:
        return _f32(w)
    if src == SRC_BF16:
        return bf16_to_f32(w)
    if src == SRC_FP8_E4M3:
        return dequant_fp8_block(w, sinv)
    raise ValueError(src)


def requant_int4_rows(w, src: int, sinv=None):
    """Checkpoint tensor -> per-row int4 (O1 after the decode)."""
    return pack_int4_row(decode_source(w, src, sinv))


def convert_int4_container(w: np.ndarray):
    """The converter's container: offset-binary codes [O][I/2] and fp32 row
    scales ([GLM-C] §06 quant_int4 with bits = 4)."""
    w = _f32(w)
    O, I = w.shape
    assert I % 2 == 0
    q = np.empty((O, I // 2), dtype=np.uint8)
    s = np.empty(O, dtype=np.float32)
    lib().orc_convert_int4_container(_p(w), O, I, _p(q), _p(s))
    return q, s


def pack_int8_row(w: np.ndarray):
    """Per-row int8 ([GLM-C] §05 quantize_rows, bits = 8): (q int8 [O][I], s [O])."""
    w = _f32(w)
    O, I = w.shape
    q = np.empty((O, I), dtype=np.int8)
    s = np.empty(O, dtype=np.float32)
    lib().orc_pack_int8_row(_p(w), O, I, _p(q), _p(s))
    return q, s


def unpack_int4_row(q: np.ndarray, I: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    O = q.shape[0]
    out = np.empty((O, I), dtype=np.int8)
    lib().orc_unpack_int4_row(_p(q), O, I, _p(out))
    return out


def dequant_int4_row(q: np.ndarray, s: np.ndarray, I: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = _f32(s)
    O = q.shape[0]
    out = np.empty((O, I), dtype=np.float64)
    lib().orc_dequant_int4_row(_p(q), _p(s), O, I, _p(out))
    return out


def pack_affine_g64(w: np.ndarray):
    w = _f32(w)
    O, I = w.shape
    assert I % 64 == 0
    q = np.empty((O, I // 2), dtype=np.uint8)
    scmn = np.empty((O, I // 64, 2), dtype=np.uint16)
    lib().orc_pack_affine_g64(_p(w), O, I, _p(q), _p(scmn))
    return q, scmn


def dequant_affine_g64(q: np.ndarray, scmn: np.ndarray, I: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scmn = np.ascontiguousarray(scmn, dtype=np.uint16)
    O = q.shape[0]
    out = np.empty((O, I), dtype=np.float64)
    lib().orc_dequant_affine_g64(_p(q), _p(scmn), O, I, _p(out))
    return out


def pack_expert(fmt: int, wg, wu, wd) -> np.ndarray:
    wg, wu, wd = _f32(wg), _f32(wu), _f32(wd)
    I, H = wg.shape
    blob = np.empty(blob_bytes(fmt, H, I), dtype=np.uint8)
    rc = lib().orc_pack_expert(fmt, H, I, _p(wg), _p(wu), _p(wd), _p(blob))
    if rc:
        raise ValueError(f"orc_pack_expert failed ({rc})")
    return blob


def dequant_expert(fmt: int, H: int, I: int, blob: np.ndarray):
    wg = np.empty((I, H), dtype=np.float64)
    wu = np.empty((I, H), dtype=np.float64)
    wd = np.empty((H, I), dtype=np.float64)
    rc = lib().orc_dequant_expert(fmt, H, I, _p(blob), _p(wg), _p(wu), _p(wd))
    if rc:
        raise ValueError(f"orc_dequant_expert failed ({rc})")
    return wg, wu, wd


def expert(fmt: int, H: int, I: int, blob: np.ndarray, x: np.ndarray):
    x = _f32(x)
    y = np.empty(H, dtype=np.float32)
    h = np.empty(I, dtype=np.float32)
    rc = lib().orc_expert(fmt, H, I, _p(blob), _p(x), _p(y), _p(h))
    if rc:
        raise ValueError(f"orc_expert failed ({rc})")
    return y, h


SCORE_SIGMOID, SCORE_SOFTMAX = 0, 1


def route(x, Wr, bias, K: int, routed_scale: float = 2.5, norm_topk: int = 1, n_group: int = 1,
          topk_group: int = 1, scoring: int = SCORE_SIGMOID):
    """Returns ids [T,K], wts [T,K], logits [T,E], scores [T,E] (sigmoid, or
    softmax probabilities), gap_k [T], gap_in [T].  With groups, gap_k is the
    smaller of the K-th/(K+1)-th score gap and the kept/excluded group-score
    gap (either closes on a near tie); with softmax scoring the gaps are
    logit differences."""
    ids, wts, logits, sig, gk, gi, gg = route_groups(x, Wr, bias, K, n_group, topk_group,
                                                      routed_scale, norm_topk, scoring)
    return ids, wts, logits, sig, np.minimum(gk, gg), gi


def route_groups(x, Wr, bias, K: int, n_group: int, topk_group: int, routed_scale: float = 2.5,
                 norm_topk: int = 1, scoring: int = SCORE_SIGMOID):
    """As route, plus gap_g [T]: the kept/excluded group-score gap."""
    x, Wr, bias = _f32(x), _f32(Wr), _f32(bias)
    T, H = x.shape
    E = Wr.shape[0]
    ids = np.empty((T, K), dtype=np.int32)
    wts = np.empty((T, K), dtype=np.float32)
    logits = np.empty((T, E), dtype=np.float32)
    sig = np.empty((T, E), dtype=np.float32)
    gk = np.empty(T, dtype=np.float64)
    gi = np.empty(T, dtype=np.float64)
    gg = np.empty(T, dtype=np.float64)
    rc = lib().orc_route_full(_p(x), T, H, _p(Wr), _p(bias), E, K, scoring, n_group, topk_group,
                              routed_scale, norm_topk, _p(ids), _p(wts), _p(logits), _p(sig),
                              _p(gk), _p(gi), _p(gg))
    if rc:
        raise ValueError(f"orc_route_full failed ({rc})")
    return ids, wts, logits, sig, gk, gi, gg


def bucket(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    cnt = np.empty(E, dtype=np.int32)
    off = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * K, dtype=np.int32)
    active = np.empty(E, dtype=np.int32)
    na = np.zeros(1, dtype=np.int32)
    rc = lib().orc_bucket(_p(ids), T, K, E, _p(cnt), _p(off), _p(perm), _p(active), _p(na))
    if rc:
        raise ValueError(f"orc_bucket failed ({rc})")
    return cnt, off, perm, active[: int(na[0])].copy()


def combine(y_routed, wts, y_shared, n_shared: int):
    y_routed, wts = _f32(y_routed), _f32(wts)
    T, K = wts.shape
    H = y_routed.shape[-1]
    ys = _f32(y_shared) if n_shared else np.zeros((1, T, H), dtype=np.float32)
    out = np.empty((T, H), dtype=np.float32)
    lib().orc_combine(T, K, H, n_shared, _p(y_routed), _p(wts), _p(ys), _p(out))
    return out


def _blob_array(blobs):
    arr = (ctypes.c_void_p * len(blobs))()
    for i, b in enumerate(blobs):
        arr[i] = None if b is None else b.ctypes.data
    return arr


def moe_layer(x, Wr, bias, K, fmt, I, blobs, shared_blobs, routed_scale=2.5, norm_topk=1,
              n_group=1, topk_group=1, scoring=SCORE_SIGMOID, shared_fmt=0):
    """Whole layer; blobs is a list of E blobs (None = not resident)."""
    x, Wr, bias = _f32(x), _f32(Wr), _f32(bias)
    T, H = x.shape
    E = Wr.shape[0]
    out = np.empty((T, H), dtype=np.float32)
    ids = np.empty((T, K), dtype=np.int32)
    wts = np.empty((T, K), dtype=np.float32)
    ba = _blob_array(blobs)
    sa = _blob_array(shared_blobs) if shared_blobs else None
    rc = lib().orc_moe_layer_full(_p(x), T, H, I, E, K, fmt, shared_fmt, _p(Wr), _p(bias), scoring,
                                  n_group,
                                  topk_group, routed_scale, norm_topk,
                                    ctypes.cast(ba, ctypes.c_void_p), len(shared_blobs or []),
                                    ctypes.cast(sa, ctypes.c_void_p) if sa is not None else None,
                                    _p(out), _p(ids), _p(wts))
    if rc:
        raise ValueError(f"orc_moe_layer failed ({rc})")
    return out, ids, wts


def rmsnorm(x, eps: float = 1e-6):
    x = _f32(x)
    T, H = x.shape
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), T, H, eps, _p(out))
    return out


def residual_layer(x, Wr, bias, K, fmt, I, blobs, shared_blobs, eps=1e-6, routed_scale=2.5,
                   norm_topk=1, n_group=1, topk_group=1, scoring=SCORE_SIGMOID, shared_fmt=0):
    """x <- x + moe(rmsnorm(x)); returns (new x, ids, wts)."""
    x = _f32(x).copy()
    T, H = x.shape
    E = Wr.shape[0]
    Wr, bias = _f32(Wr), _f32(bias)
    ids = np.empty((T, K), dtype=np.int32)
    wts = np.empty((T, K), dtype=np.float32)
    ba = _blob_array(blobs)
    sa = _blob_array(shared_blobs) if shared_blobs else None
    rc = lib().orc_residual_layer(_p(x), T, H, I, E, K, fmt, shared_fmt, _p(Wr), _p(bias),
                                  scoring, n_group, topk_group, routed_scale, norm_topk,
                                  ctypes.cast(ba, ctypes.c_void_p), len(shared_blobs or []),
                                  ctypes.cast(sa, ctypes.c_void_p) if sa is not None else None,
                                  eps, _p(ids), _p(wts))
    if rc:
        raise ValueError(f"orc_residual_layer failed ({rc})")
    return x, ids, wts
