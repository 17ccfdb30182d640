"""Workload recipes: layer shapes, seeds and value distributions.

Each entry is a synthetic stand-in for a layer of a trained model (no
checkpoint is used): expert and router weights ~N(0, 0.02), router bias
~N(0, 0.1) plus, where routing should be skewed, a Zipf(1.1) hot-expert term
of weight 0.2 over a seeded expert permutation, tokens ~N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

W_INT4_ROW = 1
W_INT4_AFFINE_G64 = 2


@dataclass(frozen=True)
class LayerConfig:
    name: str
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # routed experts
    K: int            # experts chosen per token
    n_shared: int     # always-active shared experts (same format, weight 1)
    fmt: int          # W_INT4_ROW or W_INT4_AFFINE_G64
    T: int            # tokens per forward
    n_layers: int     # layers resident (rotated, or chained)
    seed: int
    chained: bool = False     # x <- x + moe(rmsnorm(x)) between layers
    zipf_c: float = 0.0
    zipf_s: float = 1.1
    sigma_w: float = 0.02
    sigma_r: float = 0.02
    sigma_b: float = 0.1
    sigma_x: float = 1.0
    routed_scale: float = 2.5
    norm_topk: int = 1
    n_group: int = 1          # expert groups of the router (group-limited selection)
    topk_group: int = 1       # groups kept per token
    scoring: int = 0          # 0 sigmoid (+ bias selects), 1 softmax over all experts
    shared_fmt: int = 0       # shared experts' format: 0 = fmt, 3 = per-row int8
    eps: float = 1e-6

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    # tiny layer: H=512, 32 experts, top-4, I=256, one shared expert, 4 tokens
    "tiny": LayerConfig("tiny", H=512, I=256, E=32, K=4, n_shared=1, fmt=W_INT4_ROW, T=4,
                        n_layers=1, seed=0),
    # GLM-5.2-shape MoE layer, one decode token, 8 resident layers rotated
    "glm_decode": LayerConfig("glm_decode", H=6144, I=2048, E=256, K=8, n_shared=1,
                              fmt=W_INT4_ROW, T=1, n_layers=8, seed=1, zipf_c=0.2),
    # GLM-5.2 shape, 8-token speculative-verify batch through 8 chained layers
    "glm_verify": LayerConfig("glm_verify", H=6144, I=2048, E=256, K=8, n_shared=1,
                              fmt=W_INT4_ROW, T=8, n_layers=8, seed=100, chained=True,
                              zipf_c=0.2),
    # Edge0 shape, affine int4 g64, 40 chained layers, one token, top-4
    "edge0_decode": LayerConfig("edge0_decode", H=2048, I=512, E=256, K=4, n_shared=0,
                                fmt=W_INT4_AFFINE_G64, T=1, n_layers=40, seed=200, chained=True),
    # small one-token layers with a shared expert (row and affine formats):
    # shapes whose down projection and combine run as one kernel
    "mid_row": LayerConfig("mid_row", H=2048, I=256, E=32, K=4, n_shared=1, fmt=W_INT4_ROW, T=1,
                           n_layers=1, seed=400),
    "mid_affine": LayerConfig("mid_affine", H=2048, I=512, E=32, K=8, n_shared=1,
                              fmt=W_INT4_AFFINE_G64, T=1, n_layers=1, seed=401),
    # group-limited routing (8 groups of 32 experts, 4 kept, the Edge0
    # write-up's 8B setting) on small layers, row and affine formats
    "grouped_row": LayerConfig("grouped_row", H=2048, I=256, E=256, K=8, n_shared=1,
                               fmt=W_INT4_ROW, T=1, n_layers=1, seed=500, n_group=8, topk_group=4),
    "grouped_affine": LayerConfig("grouped_affine", H=2048, I=512, E=256, K=8, n_shared=0,
                                  fmt=W_INT4_AFFINE_G64, T=1, n_layers=1, seed=501, n_group=8,
                                  topk_group=4),
    # softmax scoring over all experts: renormalised weights (row format,
    # shared expert) and raw probabilities (affine, the olmoe-style step)
    "softmax_renorm": LayerConfig("softmax_renorm", H=2048, I=256, E=64, K=8, n_shared=1,
                                  fmt=W_INT4_ROW, T=1, n_layers=1, seed=700, scoring=1,
                                  routed_scale=1.0, norm_topk=1),
    "softmax_raw": LayerConfig("softmax_raw", H=2048, I=512, E=32, K=4, n_shared=0,
                               fmt=W_INT4_AFFINE_G64, T=1, n_layers=1, seed=701, scoring=1,
                               routed_scale=1.0, norm_topk=0),
    # GLM-5.2 shape prefill, 2048 tokens, one layer
    "glm_prefill": LayerConfig("glm_prefill", H=6144, I=2048, E=256, K=8, n_shared=1,
                               fmt=W_INT4_ROW, T=2048, n_layers=1, seed=300, zipf_c=0.2),
}
CONFIGS["edge0_decode_k8"] = CONFIGS["edge0_decode"].with_(name="edge0_decode_k8", K=8)
# GLM-5.2 shape decode with group-limited routing (8 groups, 4 kept), 4 layers
CONFIGS["glm_decode_grouped"] = CONFIGS["glm_decode"].with_(name="glm_decode_grouped", n_group=8,
                                                             topk_group=4, n_layers=4, seed=600)
# per-row int8 shared experts (the converted model's dense precision)
CONFIGS["int8_shared"] = CONFIGS["tiny"].with_(name="int8_shared", shared_fmt=3, seed=710)
CONFIGS["mid_int8_shared"] = CONFIGS["mid_row"].with_(name="mid_int8_shared", shared_fmt=3,
                                                      seed=711)
CONFIGS["affine_int8_shared"] = CONFIGS["mid_affine"].with_(name="affine_int8_shared", shared_fmt=3,
                                                          seed=712)
CONFIGS["glm_decode_int8_shared"] = CONFIGS["glm_decode"].with_(name="glm_decode_int8_shared",
                                                                shared_fmt=3, n_layers=4, seed=602)
# the same decode layer scored by a softmax over all experts (renormalised top-8)
CONFIGS["glm_decode_softmax"] = CONFIGS["glm_decode"].with_(name="glm_decode_softmax", scoring=1,
                                                            n_layers=4, seed=601)
# GLM-5.2 shape prefill with the shared expert in per-row int8
CONFIGS["glm_prefill_int8_shared"] = CONFIGS["glm_prefill"].with_(name="glm_prefill_int8_shared",
                                                                  shared_fmt=3, seed=303)
# GLM-5.2 shape batches of a few tokens (fresh tokens per layer), 4 layers rotated
CONFIGS["glm_batch16"] = CONFIGS["glm_decode"].with_(name="glm_batch16", T=16, n_layers=4, seed=610)
CONFIGS["glm_batch32"] = CONFIGS["glm_decode"].with_(name="glm_batch32", T=32, n_layers=4, seed=611)
