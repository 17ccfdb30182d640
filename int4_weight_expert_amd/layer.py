"""MoeLayer: a context of libmoe_int4.so with torch-tensor arguments.

PyTorch provides device memory and the stream; every step of the layer runs
in the library's HIP kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe as M


class MoeLayer:
    def __init__(self, H: int, I: int, E: int, K: int, n_shared: int, n_layers: int, fmt: int,
                 n_slots: int, max_tokens: int, routed_scale: float = 2.5, norm_topk: int = 1,
                 rms_eps: float = 1e-6, stream: torch.cuda.Stream | None = None,
                 n_group: int = 1, topk_group: int = 1, scoring: int = 0, shared_fmt: int = 0):
        self.H, self.I, self.E, self.K = H, I, E, K
        self.n_shared, self.n_layers, self.fmt = n_shared, n_layers, fmt
        self.n_slots, self.max_tokens = n_slots, max_tokens
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        cfg = M.make_config(H, I, E, K, n_shared, n_layers, fmt, n_slots, max_tokens,
                            routed_scale=routed_scale, norm_topk=norm_topk, rms_eps=rms_eps,
                            n_group=n_group, topk_group=topk_group, scoring=scoring,
                            shared_fmt=shared_fmt)
        self.ctx = M.moe_layer_create(cfg, self.stream.cuda_stream)
        self.expert_bytes = M.moe_expert_bytes(self.ctx)
        self.shared_bytes = M.lib().moe_shared_bytes(self.ctx)

    def close(self) -> None:
        if self.ctx:
            M.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- weights -----------------------------------------------------------
    def set_router(self, layer: int, W, bias) -> None:
        W = _contig_f32(W)
        bias = _contig_f32(bias)
        M.moe_set_router(self.ctx, layer, W, bias)

    def load_expert(self, slot: int, blob) -> None:
        blob = _contig_u8(blob)
        M._check("moe_load_expert", M.moe_load_expert(self.ctx, slot, blob, _nbytes(blob)))

    def pack_expert(self, slot: int, Wg, Wu, Wd) -> None:
        M._check("moe_pack_expert", M.moe_pack_expert(self.ctx, slot, Wg, Wu, Wd))

    def read_shared(self, layer: int, s: int) -> np.ndarray:
        out = np.empty(self.shared_bytes, dtype=np.uint8)
        M._check("moe_read_shared", M.moe_read_shared(self.ctx, layer, s, out, self.shared_bytes))
        return out

    def set_shared(self, layer: int, s: int, blob) -> None:
        blob = _contig_u8(blob)
        M._check("moe_set_shared", M.moe_set_shared(self.ctx, layer, s, blob, _nbytes(blob)))

    def pack_shared(self, layer: int, s: int, Wg, Wu, Wd) -> None:
        M._check("moe_pack_shared", M.moe_pack_shared(self.ctx, layer, s, Wg, Wu, Wd))

    def requant_expert(self, slot: int, src: int, Wg, Wu, Wd, sg=None, su=None, sd=None) -> None:
        """Checkpoint tensors on the device (fp32, bf16 as int16/uint16 bits, or FP8 as
        uint8 codes with fp32 block inverse scales) -> int4 in a slot."""
        M._check("moe_requant_expert",
                 M.moe_requant_expert(self.ctx, slot, src, Wg, Wu, Wd, sg, su, sd), self.ctx)

    def requant_shared(self, layer: int, s: int, src: int, Wg, Wu, Wd, sg=None, su=None,
                       sd=None) -> None:
        M._check("moe_requant_shared",
                 M.moe_requant_shared(self.ctx, layer, s, src, Wg, Wu, Wd, sg, su, sd), self.ctx)

    def import_expert(self, slot: int, qg, qu, qd, sg, su, sd) -> None:
        """The converter's container (offset-binary codes, fp32 row scales) -> a slot."""
        qg, qu, qd = (_contig_u8(a) for a in (qg, qu, qd))
        sg, su, sd = (_contig_f32(a) for a in (sg, su, sd))
        M._check("moe_import_expert", M.moe_import_expert(self.ctx, slot, qg, qu, qd, sg, su, sd),
                 self.ctx)

    def import_shared(self, layer: int, s: int, qg, qu, qd, sg, su, sd) -> None:
        qg, qu, qd = (_contig_u8(a) for a in (qg, qu, qd))
        sg, su, sd = (_contig_f32(a) for a in (sg, su, sd))
        M._check("moe_import_shared",
                 M.moe_import_shared(self.ctx, layer, s, qg, qu, qd, sg, su, sd), self.ctx)

    # ---- residency: asynchronous loads, staged slots, whole layers ----------
    def image(self, blob) -> np.ndarray:
        """Slot image of a host blob (the bytes an asynchronous load copies)."""
        return M.moe_blob_to_image(self.fmt, self.H, self.I, blob)

    def load_image_async(self, slot: int, image) -> None:
        M._check("moe_load_image_async",
                 M.moe_load_image_async(self.ctx, slot, image, _nbytes(image)), self.ctx)

    def map_async(self, layer: int, expert_ids, slots) -> None:
        M._check("moe_map_experts_async",
                 M.moe_map_experts_async(self.ctx, layer, expert_ids, slots), self.ctx)

    def load_layer_async(self, layer: int, first_slot: int, n: int, images) -> None:
        M._check("moe_load_layer_async",
                 M.moe_load_layer_async(self.ctx, layer, first_slot, n, images, _nbytes(images)),
                 self.ctx)

    def sync_copies(self) -> None:
        M._check("moe_sync_copies", M.moe_sync_copies(self.ctx), self.ctx)

    def set_staging(self, first_slot: int, per_layer: int) -> None:
        M._check("moe_set_staging", M.moe_set_staging(self.ctx, first_slot, per_layer), self.ctx)

    def stage(self, layer: int, expert_ids, images) -> int:
        """Staged executor step: returns how many images were loaded."""
        rc, n = M.moe_stage_experts(self.ctx, layer, expert_ids, images)
        M._check("moe_stage_experts", rc, self.ctx)
        return n

    def map(self, layer: int, expert_id: int, slot: int) -> None:
        M._check("moe_map_expert", M.moe_map_expert(self.ctx, layer, expert_id, slot))

    def read_slot(self, slot: int) -> np.ndarray:
        out = np.empty(self.expert_bytes, dtype=np.uint8)
        M._check("moe_read_slot", M.moe_read_slot(self.ctx, slot, out, self.expert_bytes))
        return out

    # ---- compute -----------------------------------------------------------
    def forward(self, x: torch.Tensor, layer: int, out: torch.Tensor | None = None) -> torch.Tensor:
        assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        M._check("moe_forward", M.moe_forward(self.ctx, x, T, layer, out), self.ctx)
        return out

    def forward_residual(self, x: torch.Tensor, layer: int) -> torch.Tensor:
        assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()
        M._check("moe_forward_residual", M.moe_forward_residual(self.ctx, x, x.shape[0], layer),
                 self.ctx)
        return x

    def route(self, x: torch.Tensor, layer: int):
        T = x.shape[0]
        ids = torch.empty((T, self.K), dtype=torch.int32, device=x.device)
        w = torch.empty((T, self.K), dtype=torch.float32, device=x.device)
        M._check("moe_route", M.moe_route(self.ctx, x, T, layer, ids, w), self.ctx)
        return ids, w

    def status(self):
        return M.moe_status(self.ctx)


def _contig_f32(a):
    if isinstance(a, np.ndarray):
        return np.ascontiguousarray(a, dtype=np.float32)
    return a.contiguous().float()


def _contig_u8(a):
    if isinstance(a, np.ndarray):
        return np.ascontiguousarray(a, dtype=np.uint8)
    return a.contiguous()


def _nbytes(a) -> int:
    if isinstance(a, np.ndarray):
        return a.nbytes
    return a.numel() * a.element_size()
