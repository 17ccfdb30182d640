"""ctypes binding of libmoe_int4.so (include/moe.h), argument marshalling only.

Every function has the C name and returns what the C call returns; device
buffers are passed as torch CUDA tensors (or raw integer addresses).  The
library is loaded from this package directory; if it is missing, loading
raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_int4.so")

MOE_OK = 0
MOE_E_ARG = -1
MOE_E_NOMEM = -2
MOE_E_SIZE = -3
MOE_E_SLOT = -4
MOE_E_NOT_RESIDENT = -5
MOE_E_HIP = -6
MOE_E_UNSUPPORTED = -7
MOE_E_RANGE = -8
MOE_E_BUSY = -9
MOE_E_WAIT = -10
MOE_SLOT_REMOTE = -2
MOE_W_INT4_ROW = 1
MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX = 0, 1
MOE_W_INT4_AFFINE_G64 = 2
MOE_W_INT8_ROW = 3
MOE_SRC_F32, MOE_SRC_BF16, MOE_SRC_FP8_E4M3 = 0, 1, 2

ERROR_NAMES = {0: "MOE_OK", -1: "MOE_E_ARG", -2: "MOE_E_NOMEM", -3: "MOE_E_SIZE",
               -4: "MOE_E_SLOT", -5: "MOE_E_NOT_RESIDENT", -6: "MOE_E_HIP",
               -7: "MOE_E_UNSUPPORTED", -8: "MOE_E_RANGE", -9: "MOE_E_BUSY",
               -10: "MOE_E_WAIT"}

EXPORTS = ["moe_layer_create", "moe_destroy", "moe_set_stream", "moe_expert_bytes",
           "moe_set_router", "moe_load_expert", "moe_pack_expert", "moe_set_shared",
           "moe_pack_shared", "moe_map_expert", "moe_read_slot", "moe_forward",
           "moe_forward_residual", "moe_route", "moe_status", "moe_set_gemm_min_tokens",
           "moe_set_timing", "moe_timing_summary", "moe_last_error", "moe_pack_int4_rows", "moe_pack_affine_g64",
           "moe_bucket", "moe_requant_expert", "moe_import_expert", "moe_requant_shared",
           "moe_import_shared", "moe_requant_int4_rows", "moe_requant_affine_g64",
           "moe_map_experts_async", "moe_load_image_async", "moe_load_layer_async",
           "moe_sync_copies", "moe_set_staging", "moe_stage_experts", "moe_sticky_plan",
           "moe_image_bytes", "moe_blob_to_image", "moe_requant_int8_rows", "moe_read_shared",
           "moe_shared_bytes", "moe_set_router_noalloc"]


class moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("inter", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("top_k", ctypes.c_int), ("n_shared", ctypes.c_int), ("n_layers", ctypes.c_int),
                ("wfmt", ctypes.c_int), ("n_group", ctypes.c_int), ("topk_group", ctypes.c_int),
                ("routed_scale", ctypes.c_float), ("norm_topk", ctypes.c_int),
                ("n_slots", ctypes.c_int), ("max_tokens", ctypes.c_int),
                ("rms_eps", ctypes.c_float), ("scoring", ctypes.c_int), ("shared_fmt", ctypes.c_int)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} returned {rc} ({ERROR_NAMES.get(rc, '?')})")
        self.rc = rc


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_size_t)
        sig = {
            "moe_layer_create": ([ctypes.POINTER(moe_config), vp, ctypes.POINTER(vp)], i32),
            "moe_destroy": ([vp], None),
            "moe_set_stream": ([vp, vp], i32),
            "moe_expert_bytes": ([vp], sz),
            "moe_set_router": ([vp, i32, vp, vp], i32),
            "moe_set_router_noalloc": ([vp, i32, vp, vp], i32),
            "moe_load_expert": ([vp, i32, vp, sz], i32),
            "moe_pack_expert": ([vp, i32, vp, vp, vp], i32),
            "moe_set_shared": ([vp, i32, i32, vp, sz], i32),
            "moe_pack_shared": ([vp, i32, i32, vp, vp, vp], i32),
            "moe_map_expert": ([vp, i32, i32, i32], i32),
            "moe_read_slot": ([vp, i32, vp, sz], i32),
            "moe_forward": ([vp, vp, i32, i32, vp], i32),
            "moe_forward_residual": ([vp, vp, i32, i32], i32),
            "moe_route": ([vp, vp, i32, i32, vp, vp], i32),
            "moe_status": ([vp, vp, i32, ctypes.POINTER(i32)], i32),
            "moe_set_gemm_min_tokens": ([vp, i32], i32),
            "moe_set_timing": ([vp, i32], i32),
            "moe_last_error": ([vp], ctypes.c_char_p),
            "moe_timing_summary": ([vp, vp, vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)],
                                   i32),
            "moe_pack_int4_rows": ([vp, i64, i64, vp, vp, vp], i32),
            "moe_pack_affine_g64": ([vp, i64, i64, vp, vp, vp], i32),
            "moe_bucket": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp], i32),
            "moe_requant_expert": ([vp, i32, i32, vp, vp, vp, vp, vp, vp], i32),
            "moe_import_expert": ([vp, i32, vp, vp, vp, vp, vp, vp], i32),
            "moe_requant_shared": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp], i32),
            "moe_import_shared": ([vp, i32, i32, vp, vp, vp, vp, vp, vp], i32),
            "moe_requant_int4_rows": ([vp, i32, vp, i64, i64, vp, vp, vp], i32),
            "moe_requant_affine_g64": ([vp, i32, vp, i64, i64, vp, vp, vp], i32),
            "moe_map_experts_async": ([vp, i32, i32, vp, vp], i32),
            "moe_load_image_async": ([vp, i32, vp, sz], i32),
            "moe_load_layer_async": ([vp, i32, i32, i32, vp, sz], i32),
            "moe_sync_copies": ([vp], i32),
            "moe_set_staging": ([vp, i32, i32], i32),
            "moe_stage_experts": ([vp, i32, i32, vp, vp, ctypes.POINTER(i32)], i32),
            "moe_sticky_plan": ([vp, vp, i32, vp, i32, vp, vp], i32),
            "moe_image_bytes": ([i32, i32, i32], sz),
            "moe_blob_to_image": ([i32, i32, i32, vp, sz, vp], i32),
            "moe_requant_int8_rows": ([vp, i32, vp, i64, i64, vp, vp, vp], i32),
            "moe_read_shared": ([vp, i32, i32, vp, sz], i32),
            "moe_shared_bytes": ([vp], sz),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):          # numpy host array
        return t.ctypes.data
    raise TypeError(f"cannot pass {type(t)} as a pointer")


def _check(fn: str, rc: int, ctx=None) -> int:
    if rc != MOE_OK:
        err = MoeError(fn, rc)
        if ctx and rc == MOE_E_HIP:
            err.args = (f"{err.args[0]}: {moe_last_error(ctx)}",)
        raise err
    return rc


def moe_last_error(ctx) -> str:
    return lib().moe_last_error(ctx).decode()


def make_config(H, I, E, K, n_shared, n_layers, wfmt, n_slots, max_tokens, routed_scale=2.5,
                norm_topk=1, rms_eps=1e-6, n_group=1, topk_group=1, scoring=0,
                shared_fmt=0) -> moe_config:
    return moe_config(H, I, E, K, n_shared, n_layers, wfmt, n_group, topk_group, routed_scale,
                      norm_topk, n_slots, max_tokens, rms_eps, scoring, shared_fmt)


def moe_layer_create(cfg: moe_config, stream: int = 0) -> int:
    h = ctypes.c_void_p()
    _check("moe_layer_create", lib().moe_layer_create(ctypes.byref(cfg), stream, ctypes.byref(h)))
    return h.value


def moe_layer_create_rc(cfg: moe_config, stream: int = 0) -> tuple[int, int | None]:
    h = ctypes.c_void_p()
    rc = lib().moe_layer_create(ctypes.byref(cfg), stream, ctypes.byref(h))
    return rc, h.value


def moe_destroy(ctx: int) -> None:
    lib().moe_destroy(ctx)


def moe_set_stream(ctx: int, stream: int) -> int:
    return _check("moe_set_stream", lib().moe_set_stream(ctx, stream))


def moe_expert_bytes(ctx: int) -> int:
    return int(lib().moe_expert_bytes(ctx))


def moe_set_router(ctx, layer, W, bias) -> int:
    return _check("moe_set_router", lib().moe_set_router(ctx, layer, _ptr(W), _ptr(bias)))


def moe_set_router_noalloc(ctx, layer, W, bias) -> int:
    return lib().moe_set_router_noalloc(ctx, layer, _ptr(W), _ptr(bias))


def moe_load_expert(ctx, slot, blob, nbytes) -> int:
    return lib().moe_load_expert(ctx, slot, _ptr(blob), nbytes)


def moe_pack_expert(ctx, slot, Wg, Wu, Wd) -> int:
    return lib().moe_pack_expert(ctx, slot, _ptr(Wg), _ptr(Wu), _ptr(Wd))


def moe_set_shared(ctx, layer, s, blob, nbytes) -> int:
    return lib().moe_set_shared(ctx, layer, s, _ptr(blob), nbytes)


def moe_pack_shared(ctx, layer, s, Wg, Wu, Wd) -> int:
    return lib().moe_pack_shared(ctx, layer, s, _ptr(Wg), _ptr(Wu), _ptr(Wd))


def moe_map_expert(ctx, layer, expert_id, slot) -> int:
    return lib().moe_map_expert(ctx, layer, expert_id, slot)


def moe_read_slot(ctx, slot, dst, nbytes) -> int:
    return lib().moe_read_slot(ctx, slot, _ptr(dst), nbytes)


def moe_forward(ctx, x, T, layer, out) -> int:
    return lib().moe_forward(ctx, _ptr(x), T, layer, _ptr(out))


def moe_forward_residual(ctx, x, T, layer) -> int:
    return lib().moe_forward_residual(ctx, _ptr(x), T, layer)


def moe_route(ctx, x, T, layer, ids, w) -> int:
    return lib().moe_route(ctx, _ptr(x), T, layer, _ptr(ids), _ptr(w))


def moe_status(ctx, cap: int = 4096) -> tuple[int, list[int]]:
    buf = (ctypes.c_int32 * cap)()
    n = ctypes.c_int(0)
    rc = lib().moe_status(ctx, buf, cap, ctypes.byref(n))
    return rc, [buf[i] for i in range(min(n.value, cap))]


def moe_set_gemm_min_tokens(ctx, n) -> int:
    return _check("moe_set_gemm_min_tokens", lib().moe_set_gemm_min_tokens(ctx, n))


def moe_set_timing(ctx, on: bool) -> int:
    return _check("moe_set_timing", lib().moe_set_timing(ctx, int(on)), ctx)


def moe_timing_summary(ctx, cap: int = 32) -> tuple[list[tuple[str, float]], int]:
    """[(kernel name, average ms)], number of forwards averaged."""
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    n = ctypes.c_int(0)
    nf = ctypes.c_int(0)
    _check("moe_timing_summary",
           lib().moe_timing_summary(ctx, ms, names, cap, ctypes.byref(n), ctypes.byref(nf)), ctx)
    return [(names[i].decode(), ms[i]) for i in range(min(n.value, cap))], nf.value


def moe_pack_int4_rows(w, O, I, q, s, stream=0) -> int:
    return lib().moe_pack_int4_rows(_ptr(w), O, I, _ptr(q), _ptr(s), stream)


def moe_pack_affine_g64(w, O, I, q, scmn, stream=0) -> int:
    return lib().moe_pack_affine_g64(_ptr(w), O, I, _ptr(q), _ptr(scmn), stream)


def moe_requant_expert(ctx, slot, src, Wg, Wu, Wd, sg=None, su=None, sd=None) -> int:
    return lib().moe_requant_expert(ctx, slot, src, _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(sg),
                                    _ptr(su), _ptr(sd))


def moe_import_expert(ctx, slot, qg, qu, qd, sg, su, sd) -> int:
    return lib().moe_import_expert(ctx, slot, _ptr(qg), _ptr(qu), _ptr(qd), _ptr(sg), _ptr(su),
                                   _ptr(sd))


def moe_requant_shared(ctx, layer, s, src, Wg, Wu, Wd, sg=None, su=None, sd=None) -> int:
    return lib().moe_requant_shared(ctx, layer, s, src, _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(sg),
                                    _ptr(su), _ptr(sd))


def moe_import_shared(ctx, layer, s, qg, qu, qd, sg, su, sd) -> int:
    return lib().moe_import_shared(ctx, layer, s, _ptr(qg), _ptr(qu), _ptr(qd), _ptr(sg),
                                   _ptr(su), _ptr(sd))


def moe_requant_int4_rows(w, src, sinv, O, I, q, s, stream=0) -> int:
    return lib().moe_requant_int4_rows(_ptr(w), src, _ptr(sinv), O, I, _ptr(q), _ptr(s), stream)


def moe_requant_affine_g64(w, src, sinv, O, I, q, scmn, stream=0) -> int:
    return lib().moe_requant_affine_g64(_ptr(w), src, _ptr(sinv), O, I, _ptr(q), _ptr(scmn),
                                        stream)


def moe_map_experts_async(ctx, layer, expert_ids, slots) -> int:
    ids = (ctypes.c_int * len(expert_ids))(*[int(v) for v in expert_ids])
    sl = (ctypes.c_int * len(slots))(*[int(v) for v in slots])
    return lib().moe_map_experts_async(ctx, layer, len(expert_ids), ids, sl)


def moe_load_image_async(ctx, slot, image, nbytes) -> int:
    return lib().moe_load_image_async(ctx, slot, _ptr(image), nbytes)


def moe_load_layer_async(ctx, layer, first_slot, n, images, nbytes) -> int:
    return lib().moe_load_layer_async(ctx, layer, first_slot, n, _ptr(images), nbytes)


def moe_sync_copies(ctx) -> int:
    return lib().moe_sync_copies(ctx)


def moe_set_staging(ctx, first_slot, per_layer) -> int:
    return lib().moe_set_staging(ctx, first_slot, per_layer)


def moe_stage_experts(ctx, layer, expert_ids, images) -> tuple[int, int]:
    """images: one pointer-like per id (None allowed where no load is needed)."""
    n = len(expert_ids)
    ids = (ctypes.c_int * n)(*[int(v) for v in expert_ids])
    ptrs = (ctypes.c_void_p * n)(*[_ptr(im) for im in images])
    nl = ctypes.c_int(0)
    rc = lib().moe_stage_experts(ctx, layer, n, ids, ptrs, ctypes.byref(nl))
    return rc, nl.value


def moe_sticky_plan(held, last_used, want):
    """(n_loads, slot_of, load) for the staged executor's slot choice."""
    import numpy as np
    held = np.ascontiguousarray(held, dtype=np.int32)
    last_used = np.ascontiguousarray(last_used, dtype=np.int64)
    want = np.ascontiguousarray(want, dtype=np.int32)
    slot_of = np.empty(len(want), dtype=np.int32)
    load = np.empty(len(want), dtype=np.int32)
    n = lib().moe_sticky_plan(held.ctypes.data, last_used.ctypes.data, len(held),
                              want.ctypes.data, len(want), slot_of.ctypes.data, load.ctypes.data)
    return n, slot_of, load


def moe_blob_to_image(wfmt, hidden, inter, blob):
    """Slot image (numpy uint8) of a host blob."""
    import numpy as np
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    image = np.empty_like(blob)
    _check("moe_blob_to_image", lib().moe_blob_to_image(wfmt, hidden, inter, blob.ctypes.data,
                                                        blob.nbytes, image.ctypes.data))
    return image


def moe_requant_int8_rows(w, src, sinv, O, I, q, s, stream=0) -> int:
    return lib().moe_requant_int8_rows(_ptr(w), src, _ptr(sinv), O, I, _ptr(q), _ptr(s), stream)


def moe_read_shared(ctx, layer, s, dst, nbytes) -> int:
    return lib().moe_read_shared(ctx, layer, s, _ptr(dst), nbytes)


def moe_bucket(ids, T, K, E, cnt, off, perm, active, n_active, stream=0) -> int:
    return lib().moe_bucket(_ptr(ids), T, K, E, _ptr(cnt), _ptr(off), _ptr(perm), _ptr(active),
                            _ptr(n_active), stream)
