"""Synthetic workloads: a MoeLayer filled with seeded synthetic weights.

The weights come from the seeded generator in `synth` (fp32, generated in
place in device memory) and are quantised and packed into the slot pool by
the library's own pack kernels.  Slot of (layer l, expert e) = l*E + e.
"""
from __future__ import annotations

import torch

import synth
from synth.configs import LayerConfig

from .layer import MoeLayer


def build_layer(cfg: LayerConfig, n_layers: int | None = None, max_tokens: int | None = None,
                resident=None, stream: torch.cuda.Stream | None = None) -> MoeLayer:
    """resident(layer, expert) -> bool picks which experts get a slot (all by default)."""
    L = cfg.n_layers if n_layers is None else n_layers
    Tm = cfg.T if max_tokens is None else max_tokens
    ml = MoeLayer(cfg.H, cfg.I, cfg.E, cfg.K, cfg.n_shared, L, cfg.fmt, n_slots=L * cfg.E,
                  max_tokens=Tm, routed_scale=cfg.routed_scale, norm_topk=cfg.norm_topk,
                  rms_eps=cfg.eps, stream=stream, n_group=cfg.n_group, topk_group=cfg.topk_group,
                  scoring=cfg.scoring, shared_fmt=cfg.shared_fmt)
    dev = torch.device("cuda", torch.cuda.current_device())
    n = cfg.I * cfg.H
    wg = torch.empty(n, dtype=torch.float32, device=dev)
    wu = torch.empty(n, dtype=torch.float32, device=dev)
    wd = torch.empty(n, dtype=torch.float32, device=dev)
    st = ml.stream.cuda_stream
    for layer in range(L):
        ml.set_router(layer, synth.router_weight(cfg, layer), synth.router_bias(cfg, layer))
        for e in list(range(cfg.E)) + [cfg.E + s for s in range(cfg.n_shared)]:
            if e < cfg.E and resident is not None and not resident(layer, e):
                continue
            kg, ku, kd = synth.expert_keys(cfg, layer, e)
            synth.gpu_fill_gauss(wg.data_ptr(), n, kg, cfg.sigma_w, 0, st)
            synth.gpu_fill_gauss(wu.data_ptr(), n, ku, cfg.sigma_w, 0, st)
            synth.gpu_fill_gauss(wd.data_ptr(), n, kd, cfg.sigma_w, 0, st)
            if e < cfg.E:
                slot = layer * cfg.E + e
                ml.pack_expert(slot, wg, wu, wd)
                ml.map(layer, e, slot)
            else:
                ml.pack_shared(layer, e - cfg.E, wg, wu, wd)
    torch.cuda.synchronize()
    return ml


def tokens_device(cfg: LayerConfig, T: int | None = None, stream: int = 0) -> torch.Tensor:
    x = synth.tokens(cfg, T=T, stream=stream)
    return torch.from_numpy(x).cuda()
