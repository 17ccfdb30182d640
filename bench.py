#!/usr/bin/env python3
"""Benchmark of the int4 MoE FFN step on one MI355X.

Step = one moe_forward of a GLM-5.2-shape MoE layer (H=6144, 256 experts,
top-8, I=2048, one shared expert, int4 per-row scales) on one decode token,
rotating through 8 resident layers (38.7 GB of experts in the slot pool, so
the 256 MB Infinity Cache cannot serve repeats).  Inputs are resident in HBM
before the timed region.  Prints one JSON line.

The timed region is one replay of a HIP graph holding exactly --steps
forwards (layers in turn), bracketed by a full synchronisation and events;
the headline is the median over several such replays.  Also measured
(under "extra"): a streaming-read probe (the HBM read rate this part
reaches), the 8-token speculative-verify batch through 8 chained layers,
the Edge0-shape 40-layer decode step (affine int4 g64, top-4 and top-8), the
2048-token prefill layer and the variants of the decode layer; and the CPU
oracle on bounded samples of each workload, one thread and all host cores
(cpu_baseline, and extra.cpu_baseline_by_workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, datasheet


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def expert_bytes(cfg, fmt: int) -> int:
    """One expert's codes and scales in format fmt (1 int4 row, 2 int4
    affine g64, 3 int8 row)."""
    if fmt == 1:
        return 3 * cfg.H * cfg.I // 2 + 4 * (2 * cfg.I + cfg.H)
    if fmt == 3:
        return 3 * cfg.H * cfg.I + 4 * (2 * cfg.I + cfg.H)
    return 3 * cfg.H * cfg.I // 2 + 12 * cfg.H * cfg.I // 64


def glm_bytes(cfg, n_routed_read: int, T: int) -> int:
    """Algorithmic HBM bytes of one layer forward: router weights and bias,
    every routed expert read once and the shared experts (codes + scales),
    tokens in and out."""
    shared = cfg.n_shared * expert_bytes(cfg, cfg.shared_fmt or cfg.fmt)
    return (cfg.E * cfg.H * 4 + cfg.E * 4 + n_routed_read * expert_bytes(cfg, cfg.fmt) + shared
            + 2 * T * cfg.H * 4)


def gateup_unit_bytes(cfg) -> int:
    """Algorithmic bytes of one expert's gate and up matrices (codes + scales)."""
    if cfg.fmt == 1:
        return 2 * (cfg.I * cfg.H // 2) + 2 * 4 * cfg.I
    return 2 * (cfg.I * cfg.H // 2) + 2 * 4 * cfg.I * (cfg.H // 64)


def time_graph(torch, ml, step_fns, steps: int, warmup: int, replays: int = 5):
    """Captures exactly `steps` step calls (step_fns[i % len], so the
    resident layers rotate) into one HIP graph and times `replays` replays
    of it, each bracketed by events on the replay stream after a full
    synchronisation.  Returns (graph, median seconds per step, stats): the
    headline is the median replay divided by `steps`; the stats also carry
    p10/p90 and the host wall clock of each bracketed replay."""
    import numpy as np
    from int4_weight_expert_amd import moe as M
    L = len(step_fns)
    for i in range(warmup):
        step_fns[i % L]()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    M.moe_set_stream(ml.ctx, cap.cuda_stream)
    try:
        with torch.cuda.graph(g, stream=cap):
            for i in range(steps):
                step_fns[i % L]()
    finally:
        M.moe_set_stream(ml.ctx, torch.cuda.current_stream().cuda_stream)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    ev, wall = [], []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        wall.append(time.perf_counter() - t0)
        ev.append(a.elapsed_time(b) * 1e-3)
    per = np.array(ev) / steps
    stats = {"steps_per_replay": steps, "replays": replays,
             "median_us_per_step": float(np.median(per)) * 1e6,
             "p10_us_per_step": float(np.quantile(per, 0.1)) * 1e6,
             "p90_us_per_step": float(np.quantile(per, 0.9)) * 1e6,
             "wall_us_per_step_mean": float(np.mean(wall)) / steps * 1e6}
    return g, float(np.median(per)), stats


def time_eager(torch, step_fns, steps: int):
    L = len(step_fns)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_fns[i % L]()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def kernel_times(torch, ml, step_fns, steps: int):
    """Average per-kernel durations from the library's marker events on its
    stream over `steps` eager forwards; a short GPU sleep first lets the host
    queue run ahead, so that the markers bracket kernels, not host gaps."""
    from int4_weight_expert_amd import moe as M
    L = len(step_fns)
    torch.cuda.synchronize()
    M.moe_set_timing(ml.ctx, True)
    torch.cuda._sleep(50_000_000)
    for i in range(steps):
        step_fns[i % L]()
    summary, nf = M.moe_timing_summary(ml.ctx)
    M.moe_set_timing(ml.ctx, False)
    torch.cuda.synchronize()
    return dict(summary), nf


def bench_decode(torch, args, result):
    import synth
    from int4_weight_expert_amd import workload
    cfg = synth.CONFIGS["glm_decode"]
    log(f"[bench] building {cfg.name}: {cfg.n_layers} layers x {cfg.E} experts")
    ml = workload.build_layer(cfg, max_tokens=8)
    L = cfg.n_layers
    xs = [workload.tokens_device(cfg, T=1, stream=l) for l in range(L)]
    outs = [torch.empty_like(x) for x in xs]
    fns = [(lambda l=l: ml.forward(xs[l], l, outs[l])) for l in range(L)]
    eager_ref = []
    for l in range(L):
        fns[l]()
        eager_ref.append(outs[l].clone())
    g, t_graph, pct = time_graph(torch, ml, fns, args.steps, args.warmup,
                                 replays=max(5, -(-400 // args.steps)))
    n_timed = args.steps
    graph_ok = all(torch.equal(outs[l], eager_ref[l]) for l in range(L))
    t_eager = time_eager(torch, fns, args.steps)
    kt, nf = kernel_times(torch, ml, fns, args.steps)
    rc, missing = ml.status()
    if rc != 0:
        raise RuntimeError(f"status {rc} {missing}")
    t_step = t_graph if graph_ok else t_eager
    n_gateup = cfg.K + cfg.n_shared
    alg_gateup = n_gateup * gateup_unit_bytes(cfg)
    t_gu = kt["gateup_gemv"] * 1e-3
    layer_bytes = glm_bytes(cfg, cfg.K, 1)
    result.update({
        "metric": "MoE-FFN tokens/s (GLM-shape layer, T=1 decode)",
        "value": 1.0 / t_step,
        "unit": "tokens/s",
        "ms_per_step": t_step * 1e3,
        "steps": n_timed,
        "roofline": {
            "bound": "hbm", "achieved": alg_gateup / t_gu / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": alg_gateup / t_gu / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "kernel": "k_gu8 (one-token int4 gate/up: a workgroup per (expert, 8 rows), "
                      "4 wavefronts splitting H, h written directly)",
            "algorithmic_bytes_per_launch": alg_gateup,
            "avg_launch_ms": kt["gateup_gemv"],
        },
    })
    result["extra"]["glm_decode"] = {
        "us_per_layer_graph": t_graph * 1e6, "us_per_layer_eager": t_eager * 1e6,
        "graph_replay_percentiles": pct,
        "graph_replay_matches_eager": graph_ok,
        "layer_algorithmic_bytes": layer_bytes,
        "layer_gbps": layer_bytes / t_step / 1e9,
        "layer_frac_hbm_peak": layer_bytes / t_step / 1e9 / HBM_PEAK_GBS,
        "kernel_avg_ms": kt, "kernel_timing_forwards": nf,
    }
    log(f"[bench] glm_decode: {t_step * 1e6:.1f} us/layer (graph {t_graph * 1e6:.1f}, eager "
        f"{t_eager * 1e6:.1f}); kernels {kt}")
    ml.close()
    del ml, xs, outs
    torch.cuda.empty_cache()


def bench_rotated(torch, name, steps, result):
    """One-token forwards rotated over the resident layers (as the decode
    bench), graph-replayed: per-layer time and percentiles."""
    import synth
    from int4_weight_expert_amd import workload
    cfg = synth.CONFIGS[name]
    log(f"[bench] building {name}: {cfg.n_layers} layers x {cfg.E} experts")
    ml = workload.build_layer(cfg, max_tokens=8)
    L = cfg.n_layers
    xs = [workload.tokens_device(cfg, T=1, stream=l) for l in range(L)]
    outs = [torch.empty_like(x) for x in xs]
    fns = [(lambda l=l: ml.forward(xs[l], l, outs[l])) for l in range(L)]
    for fn in fns:
        fn()
    g, t, pct = time_graph(torch, ml, fns, steps, 20)
    layer_bytes = glm_bytes(cfg, cfg.K, 1)
    result["extra"][name] = {
        "T": 1, "layers": L, "n_group": cfg.n_group, "topk_group": cfg.topk_group,
        "scoring": "softmax" if cfg.scoring else "sigmoid",
        "shared_format": "int8 row" if cfg.shared_fmt == 3 else "as routed",
        "us_per_layer": t * 1e6, "graph_replay_percentiles": pct,
        "layer_algorithmic_bytes": layer_bytes, "layer_gbps": layer_bytes / t / 1e9,
        "layer_frac_hbm_peak": layer_bytes / t / 1e9 / HBM_PEAK_GBS,
    }
    log(f"[bench] {name}: {t * 1e6:.1f} us/layer, {layer_bytes / t / 1e9:.0f} GB/s")
    ml.close()
    del ml, xs, outs
    torch.cuda.empty_cache()


def bench_requant(torch, result, n_experts: int = 32, steps: int = 256):
    """The converter step on the device: FP8 E4M3 GLM-5.2-shape experts
    (gate/up [2048, 6144], down [6144, 2048], one fp32 inverse scale per
    128 x 128 block) requantised to int4 straight into slots, one launch per
    expert, graph-replayed over n_experts distinct sources (1.2 GB, beyond the
    Infinity Cache)."""
    import numpy as np
    import synth
    from int4_weight_expert_amd import moe as M
    from int4_weight_expert_amd.layer import MoeLayer
    H, I = 6144, 2048
    log(f"[bench] requant: {n_experts} FP8 experts H={H} I={I}")
    ml = MoeLayer(H, I, 256, 8, 0, 1, M.MOE_W_INT4_ROW, n_slots=n_experts, max_tokens=1)
    tmp = torch.empty(H * I, dtype=torch.float32, device="cuda")
    srcs = []
    for e in range(n_experts):
        mats = []
        for t, (O, In) in enumerate([(I, H), (I, H), (H, I)]):
            k = synth.key(800, 0, t, e)
            synth.gpu_fill_gauss(tmp.data_ptr(), O * In, k, 112.0, 0,
                                 torch.cuda.current_stream().cuda_stream)
            q = tmp.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).clone()
            nb = ((O + 127) // 128) * ((In + 127) // 128)
            si = (0.02 * 4 / 448 * np.exp(synth.gauss(k, nb, 0.3, idx0=O * In)
                                          .astype(np.float64))).astype(np.float32)
            mats.append((q, torch.from_numpy(si).cuda()))
        srcs.append(mats)
    del tmp
    fns = [(lambda e=e: ml.requant_expert(e, M.MOE_SRC_FP8_E4M3, srcs[e][0][0], srcs[e][1][0],
                                          srcs[e][2][0], srcs[e][0][1], srcs[e][1][1],
                                          srcs[e][2][1])) for e in range(n_experts)]
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    first = ml.read_slot(0)
    g, t, _ = time_graph(torch, ml, fns, steps, n_experts)
    assert np.array_equal(ml.read_slot(0), first), "graph replay changed a slot"
    read_b = 3 * H * I + 4 * (2 * (I // 128) * (H // 128) + (H // 128) * (I // 128))
    write_b = 3 * H * I // 2 + 4 * (2 * I + H)
    result["extra"]["requant_fp8_glm_expert"] = {
        "experts": n_experts, "us_per_expert": t * 1e6, "algorithmic_bytes": read_b + write_b,
        "read_bytes": read_b, "write_bytes": write_b,
        "gbps": (read_b + write_b) / t / 1e9,
        "frac_hbm_peak": (read_b + write_b) / t / 1e9 / HBM_PEAK_GBS,
        "experts_per_s": 1.0 / t,
    }
    log(f"[bench] requant: {t * 1e6:.1f} us/expert, {(read_b + write_b) / t / 1e9:.0f} GB/s")
    ml.close()
    del ml, srcs, g
    torch.cuda.empty_cache()


def bench_staged(torch, result, n_layers: int = 8, per_layer: int = 16, n_tokens: int = 64):
    """The staged executor on the Edge0 shape (H=2048, I=512, 256 affine
    experts, top-4): every layer-step stages the experts its token routes to
    (sticky slots, loads of slot images from pinned host memory on the copy
    stream) and runs the layer.  Reported beside it: the same loads alone
    and the same forwards with every expert resident, so the overlap of
    copies and compute shows."""
    import numpy as np
    import synth
    from int4_weight_expert_amd import moe as M
    from int4_weight_expert_amd.layer import MoeLayer
    cfg = synth.CONFIGS["edge0_decode"]
    H, I, E, K, L = cfg.H, cfg.I, cfg.E, cfg.K, n_layers
    log(f"[bench] staged: building {L} x {E} Edge0 slot images in pinned memory")
    src = MoeLayer(H, I, E, K, 0, 1, cfg.fmt, n_slots=1, max_tokens=1)
    nb = src.expert_bytes
    images = torch.empty((L, E, nb), dtype=torch.uint8, pin_memory=True)
    n = I * H
    w = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    st = torch.cuda.current_stream().cuda_stream
    for l in range(L):
        for e in range(E):
            for t, k in enumerate(synth.expert_keys(cfg, l, e)):
                synth.gpu_fill_gauss(w[t].data_ptr(), n, k, cfg.sigma_w, 0, st)
            src.pack_expert(0, *w)
            images[l, e].numpy()[:] = src.image(src.read_slot(0))
    src.close()
    del w
    # routing of every (token, layer) from the routers alone
    ml = MoeLayer(H, I, E, K, 0, L, cfg.fmt, n_slots=L * per_layer, max_tokens=n_tokens)
    full = MoeLayer(H, I, E, K, 0, L, cfg.fmt, n_slots=L * E, max_tokens=n_tokens)
    xs = []
    ids = np.empty((L, n_tokens, K), dtype=np.int32)
    for l in range(L):
        Wr, br = synth.router_weight(cfg, l), synth.router_bias(cfg, l)
        ml.set_router(l, Wr, br)
        full.set_router(l, Wr, br)
        x = torch.from_numpy(synth.tokens(cfg, T=n_tokens, stream=500 + l)).cuda()
        xs.append(x)
        ids[l] = ml.route(x, l)[0].cpu().numpy()
        full.load_layer_async(l, l * E, E, images[l])
    full.sync_copies()
    ptrs = [[images[l, e].data_ptr() for e in range(E)] for l in range(L)]
    outs = [torch.empty((1, H), dtype=torch.float32, device="cuda") for _ in range(L)]

    def staged(run_forward=True, run_stage=True, ctx=ml):
        loads = 0
        for t in range(n_tokens):
            for l in range(L):
                want = sorted(set(ids[l, t].tolist()))
                if run_stage:
                    loads += ctx.stage(l, want, [ptrs[l][e] for e in want])
                if run_forward:
                    ctx.forward(xs[l][t:t + 1], l, outs[l])
        return loads

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = fn()
        t_host = time.perf_counter() - t0
        ml.sync_copies()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, t_host, r

    def reset():
        ml.set_staging(0, per_layer)
        for l in range(L):     # the staged slots leave the table: the next run starts cold
            ml.map_async(l, list(range(E)), [-1] * E)
        torch.cuda.synchronize()

    steps = n_tokens * L
    ml.set_staging(0, per_layer)
    timed(lambda: staged())                       # warm-up (events, first touches)
    reset()
    t_both, t_host, loads = timed(lambda: staged())
    t_comp, t_host_c, _ = timed(lambda: staged(run_stage=False, ctx=full))
    # the same number of slot-image copies as raw pinned copies on two streams
    dst = torch.empty((2, nb), dtype=torch.uint8, device="cuda")
    ss = [torch.cuda.Stream(), torch.cuda.Stream()]
    flat = images.view(L * E, nb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(loads):
        with torch.cuda.stream(ss[i % 2]):
            dst[i % 2].copy_(flat[(i * 97) % (L * E)], non_blocking=True)
    torch.cuda.synchronize()
    t_plain = time.perf_counter() - t0
    del dst
    bytes_loaded = loads * nb
    out = {
        "layers": L, "tokens": n_tokens, "per_layer_slots": per_layer, "expert_bytes": nb,
        "loads_per_layer_step": loads / steps, "sticky_hit_rate": 1 - loads / (steps * K),
        "us_per_layer_staged": t_both / steps * 1e6,
        "us_per_layer_resident": t_comp / steps * 1e6,
        "us_per_layer_plain_copies": t_plain / steps * 1e6,
        "host_enqueue_us_per_layer_staged": t_host / steps * 1e6,
        "host_enqueue_us_per_layer_resident": t_host_c / steps * 1e6,
        "h2d_gbps_staged": bytes_loaded / t_both / 1e9,
        "h2d_gbps_plain_copies": bytes_loaded / t_plain / 1e9,
        "copy_hidden_frac": max(0.0, min(1.0, (t_plain + t_comp - t_both) / min(t_plain, t_comp))),
    }
    result["extra"]["staged_edge0"] = out
    log(f"[bench] staged: {out['us_per_layer_staged']:.1f} us/layer-step (host enqueue "
        f"{out['host_enqueue_us_per_layer_staged']:.1f}; plain copies "
        f"{out['us_per_layer_plain_copies']:.1f}, resident {out['us_per_layer_resident']:.1f}), "
        f"{out['loads_per_layer_step']:.2f} loads/step, {out['h2d_gbps_staged']:.1f} GB/s H2D")
    ml.close()
    full.close()
    del images, ml, full
    torch.cuda.empty_cache()


def bench_batch(torch, name, steps, result):
    """A batch of a few tokens per forward (fresh tokens for each of the
    resident layers, taken in turn), graph-replayed: per-layer time and the
    HBM rate over the distinct experts the layers read."""
    import numpy as np
    import synth
    from int4_weight_expert_amd import workload
    cfg = synth.CONFIGS[name]
    log(f"[bench] building {name}: {cfg.n_layers} layers x {cfg.E} experts, T={cfg.T}")
    ml = workload.build_layer(cfg, max_tokens=cfg.T)
    L = cfg.n_layers
    xs = [workload.tokens_device(cfg, T=cfg.T, stream=l) for l in range(L)]
    outs = [torch.empty_like(x) for x in xs]
    distinct = [len(np.unique(ml.route(xs[l], l)[0].cpu().numpy())) for l in range(L)]
    fns = [(lambda l=l: ml.forward(xs[l], l, outs[l])) for l in range(L)]
    for fn in fns:
        fn()
    g, t, pct = time_graph(torch, ml, fns, steps, 8)
    bytes_layer = float(np.mean([glm_bytes(cfg, u, cfg.T) for u in distinct]))
    result["extra"][name] = {
        "T": cfg.T, "layers": L, "us_per_layer": t * 1e6, "graph_replay_percentiles": pct,
        "tokens_per_s": cfg.T / t, "distinct_experts_per_layer": distinct,
        "layer_algorithmic_bytes_mean": bytes_layer, "layer_gbps": bytes_layer / t / 1e9,
        "layer_frac_hbm_peak": bytes_layer / t / 1e9 / HBM_PEAK_GBS,
    }
    log(f"[bench] {name}: {t * 1e6:.1f} us/layer, {bytes_layer / t / 1e9:.0f} GB/s over "
        f"{np.mean(distinct):.0f} distinct experts")
    ml.close()
    del ml, xs, outs
    torch.cuda.empty_cache()


def bench_chain(torch, name, steps, result):
    """Chained residual layers (x <- x + moe(rmsnorm(x))): per-layer time."""
    import numpy as np
    import synth
    from int4_weight_expert_amd import workload
    cfg = synth.CONFIGS[name]
    log(f"[bench] building {name}: {cfg.n_layers} layers x {cfg.E} experts, T={cfg.T}")
    ml = workload.build_layer(cfg)
    L = cfg.n_layers
    x0 = workload.tokens_device(cfg, T=cfg.T)
    x = x0.clone()
    distinct = []
    for l in range(L):      # routing of the chain, for the byte count
        ids, _ = ml.route(x, l)
        distinct.append(len(np.unique(ids.cpu().numpy())))
        ml.forward_residual(x, l)
    fns = [(lambda l=l: ml.forward_residual(x, l)) for l in range(L)]
    reps = max(1, steps // L)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        x.copy_(x0)
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / (reps * L)
    x.copy_(x0)
    g, t_graph, pct = time_graph(torch, ml, fns, reps * L, 0)
    t = t_graph
    x.copy_(x0)
    bytes_layer = float(np.mean([glm_bytes(cfg, u, cfg.T) for u in distinct]))
    result["extra"][name] = {
        "T": cfg.T, "layers": L, "us_per_layer": t * 1e6, "us_per_layer_eager": t_eager * 1e6,
        "graph_replay_percentiles": pct,
        "us_per_step_all_layers": t * L * 1e6, "tokens_per_s_per_layer": cfg.T / t,
        "distinct_experts_per_layer": distinct,
        "layer_algorithmic_bytes_mean": bytes_layer,
        "layer_gbps": bytes_layer / t / 1e9, "layer_frac_hbm_peak": bytes_layer / t / 1e9 / HBM_PEAK_GBS,
    }
    log(f"[bench] {name}: {t * 1e6:.1f} us/layer (eager {t_eager * 1e6:.1f}), "
        f"{bytes_layer / t / 1e9:.0f} GB/s")
    ml.close()
    del ml
    torch.cuda.empty_cache()


def bench_prefill(torch, steps, result, name="glm_prefill"):
    import numpy as np
    import synth
    from int4_weight_expert_amd import workload
    cfg = synth.CONFIGS[name]
    log(f"[bench] building {name}: T={cfg.T}")
    ml = workload.build_layer(cfg)
    x = workload.tokens_device(cfg)
    out = torch.empty_like(x)
    ids, _ = ml.route(x, 0)
    ids_np = ids.cpu().numpy()
    distinct = len(np.unique(ids_np))
    counts = np.bincount(ids_np.ravel(), minlength=cfg.E)
    tiles = int(np.sum((counts + 127) // 128) + cfg.n_shared * ((cfg.T + 127) // 128))
    rows = int(counts.sum() + cfg.n_shared * cfg.T)
    sizes = np.concatenate([counts[counts > 0], np.full(cfg.n_shared, cfg.T)])
    issued = int(np.sum((sizes // 128) * 128 + ((sizes % 128 + 31) // 32) * 32))  # 32-row blocks
    ml.forward(x, 0, out)
    torch.cuda.synchronize()
    eager_out = out.clone()
    n = max(2, steps)
    t0 = time.perf_counter()
    for _ in range(n):
        ml.forward(x, 0, out)
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / n
    # one forward captured in a HIP graph and replayed (as the decode bench)
    g, t, pct = time_graph(torch, ml, [lambda: ml.forward(x, 0, out)], n, 2)
    graph_ok = bool(torch.equal(out, eager_out))
    if not graph_ok:
        t = t_eager
    kt, _ = kernel_times(torch, ml, [lambda: ml.forward(x, 0, out)], 3)
    flops = 2.0 * (cfg.T * cfg.K + cfg.T * cfg.n_shared) * 3 * cfg.H * cfg.I
    result["extra"][name] = {
        "T": cfg.T, "shared_format": "int8 row" if cfg.shared_fmt == 3 else "as routed",
        "ms_per_layer": t * 1e3, "ms_per_layer_eager": t_eager * 1e3,
        "graph_replay_matches_eager": graph_ok, "graph_replay_percentiles": pct, "tokens_per_s": cfg.T / t,
        "expert_flops": flops, "tflops": flops / t / 1e12,
        "frac_fp16_mfma_peak": flops / t / 1e12 / BF16_PEAK_TFLOPS,
        "distinct_experts": distinct, "kernel_avg_ms": kt,
        "tokens_per_expert_max": int(counts.max()), "gemm_tiles_128": tiles,
        "gemm_row_occupancy": rows / (tiles * 128.0), "gemm_rows_issued_32": issued,
        "gemm_issued_row_occupancy": rows / float(issued),
    }
    log(f"[bench] {name}: {t * 1e3:.2f} ms/layer, {flops / t / 1e12:.1f} TFLOP/s; {kt}")
    ml.close()
    del ml
    torch.cuda.empty_cache()


def copy_probe(torch, result):
    """A plain device-to-device copy of known size (256 MiB read, 256 MiB
    written, five times): the calibration kernel for the HBM byte counters."""
    n = 64 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    result["extra"]["copy_probe"] = {"bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4,
                                     "copies": 5}
    del src, dst
    torch.cuda.empty_cache()


def stream_ceiling(torch, result, unit_bytes: int):
    """The HBM read rate a plain streaming kernel reaches here (the
    achievable ceiling the byte-bound kernels are held against): reads of
    `unit_bytes` (the decode gate/up launch's algorithmic bytes) rotated
    over 16 disjoint windows of a 2 GiB buffer, so that the 256 MB Infinity
    Cache cannot serve repeats, and reads of the whole 2 GiB; grid sizes and
    plain or non-temporal loads swept, each launch timed with events on the
    current stream (median of 48)."""
    import ctypes
    import numpy as np
    lib = ctypes.CDLL(os.path.join(ROOT, "int4_weight_expert_amd", "libhbm_probe.so"))
    lib.hbm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    lib.hbm_probe_read.restype = ctypes.c_int
    total = 2 << 30
    buf = torch.full((total,), 0x5A, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    unit = unit_bytes // 4096 * 4096
    win = total // 16

    def run(nbytes, blocks, nt, n=48, rotate=True):
        evs = []
        for i in range(n):
            off = (i % 16) * win if rotate else 0
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            rc = lib.hbm_probe_read(buf.data_ptr() + off, nbytes, blocks, nt, sink.data_ptr(),
                                    0xDEADBEEF, st.cuda_stream)
            b.record(st)
            if rc != 0:
                raise RuntimeError(f"hbm_probe_read: hip error {rc}")
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = np.median([a.elapsed_time(b) for a, b in evs])
        return nbytes / (ms * 1e-3) / 1e9, float(ms)

    rows = []
    for nt in (0, 1):
        for blocks in (1024, 2048, 4096, 8192):
            gbs, ms = run(unit, blocks, nt)
            rows.append({"bytes": unit, "rotated_windows": 16, "blocks": blocks,
                         "nontemporal": bool(nt), "gbps": gbs, "median_ms": ms})
    best = max(rows, key=lambda r: r["gbps"])
    gbs_all, ms_all = run(total, best["blocks"], int(best["nontemporal"]), n=8, rotate=False)
    # the one-token gate/up kernel's workgroups (8 rows each) reading 9 GLM
    # experts' gate and up codes in 64-row blocks (a slot layout where their
    # pieces interleave) and in 8-row groups (contiguous per workgroup, the
    # slot layout used), rotated over 12 disjoint sets of 9 slots
    lib.hbm_probe_pattern.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    lib.hbm_probe_pattern.restype = ctypes.c_int
    exp_bytes, n_exp = 18915328, 9
    pat = {}
    for pattern, name in ((0, "rows8_of_64row_blocks"), (2, "rows8_of_64row_blocks_xcd_order"),
                          (1, "rows8_groups_contiguous")):
        evs = []
        for i in range(48):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            rc = lib.hbm_probe_pattern(buf.data_ptr() + (i % 12) * n_exp * exp_bytes, exp_bytes,
                                       n_exp, pattern, sink.data_ptr(), 0xDEADBEEF, st.cuda_stream)
            b.record(st)
            if rc != 0:
                raise RuntimeError(f"hbm_probe_pattern: hip error {rc}")
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        pat[name] = {"gbps": n_exp * 256 * 49152 / (ms * 1e-3) / 1e9, "median_ms": ms}
    out = {"unit_reads": rows, "best_unit_gbps": best["gbps"],
           "whole_2gib_gbps": gbs_all, "whole_2gib_ms": ms_all,
           "ceiling_gbps": max(best["gbps"], gbs_all), "access_pattern": pat}
    result["extra"]["hbm_stream_probe"] = out
    log(f"[bench] streaming-read ceiling: {best['gbps']:.0f} GB/s for {unit} B reads "
        f"({best['blocks']} blocks, nt={best['nontemporal']}), {gbs_all:.0f} GB/s whole 2 GiB; "
        f"8 rows of 64-row blocks {pat['rows8_of_64row_blocks']['gbps']:.0f} GB/s "
        f"({pat['rows8_of_64row_blocks_xcd_order']['gbps']:.0f} XCD-grouped), 8-row groups (contiguous) "
        f"{pat['rows8_groups_contiguous']['gbps']:.0f} GB/s")
    del buf, sink
    torch.cuda.empty_cache()
    return out["ceiling_gbps"]


def measured_traffic():
    """HBM bytes per launch of the one-token gate/up kernel from the
    committed counter runs, if they were taken on the current kernel source
    (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "int4_weight_expert_amd", "csrc", "k_tok1.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("k_tok1_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def _oracle_rate(jobs, threads: int):
    """Times the oracle over jobs [(OracleLayer, x [T,H], residual)], one
    token per call, on `threads` host threads (each oracle call is
    single-threaded C and releases the interpreter lock).  Returns
    (token-layers, seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    calls = []
    for ref, x, residual in jobs:
        cfg = ref.cfg
        blobs = [ref.cache.get(e) for e in range(cfg.E)]
        for t in range(x.shape[0]):
            calls.append((ref, cfg, blobs, x[t:t + 1], residual))

    def one(c):
        ref, cfg, blobs, xt, residual = c
        if residual:
            oracle.residual_layer(xt, ref.W, ref.b, cfg.K, cfg.fmt, cfg.I, blobs, ref.shared,
                                  cfg.eps, cfg.routed_scale, cfg.norm_topk)
        else:
            oracle.moe_layer(xt, ref.W, ref.b, cfg.K, cfg.fmt, cfg.I, blobs, ref.shared)

    t0 = time.perf_counter()
    if threads == 1:
        for c in calls:
            one(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, calls))
    return len(calls), time.perf_counter() - t0


def _oracle_jobs(cfg, layers, T, stream0, residual=False):
    """Routes each sample on the oracle and packs the experts it selects
    (not timed)."""
    import oracle
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import OracleLayer
    jobs = []
    for l in layers:
        ref = OracleLayer(cfg, l)
        x = synth.tokens(cfg, T=T, stream=stream0 + l)
        xin = oracle.rmsnorm(x, cfg.eps) if residual else x
        ids, *_ = ref.route(xin)
        ref.need(ids)
        jobs.append((ref, x, residual))
    return jobs


def cpu_baseline(n_tok: int):
    """The oracle, as it stands, on bounded samples of each workload, timed
    on this host (forward only: routing for the sample and expert packing
    happen before the clock starts).  Returns (the headline entry for the
    decode workload, per-workload entries)."""
    import synth
    nproc = min(16, os.cpu_count() or 1)
    host = {"host_cpu": _cpu_model(), "host_nproc": os.cpu_count()}
    out = {}
    # GLM decode (T = 1): n_tok token-layers over the 8 layers, one thread
    cfg = synth.CONFIGS["glm_decode"]
    per = max(1, n_tok // cfg.n_layers)
    jobs = _oracle_jobs(cfg, range(cfg.n_layers), per, 1000)
    n, dt = _oracle_rate(jobs, 1)
    head = {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} token-layers (T=1) of the 8-layer GLM decode workload ({per} tokens "
                      f"per layer), single-threaded C oracle, fp64 accumulate; expert packing "
                      f"excluded; {dt:.1f} s", **host}
    # the same workload on every host core: P threads over a larger sample
    jobs_p = _oracle_jobs(cfg, [0], 6 * nproc, 2000)
    n, dt = _oracle_rate(jobs_p, nproc)
    out["glm_decode_all_cores"] = {"value": n / dt, "unit": "tokens/s", "cores": nproc,
                                   "sample": f"{n} tokens (T=1 each) through layer 0 of the GLM "
                                             f"decode workload, {nproc} threads, {dt:.1f} s"}
    # GLM verify (T = 8 x 8 chained layers): 2 of the 8 layers, scaled to the stack
    cfg = synth.CONFIGS["glm_verify"]
    jobs = _oracle_jobs(cfg, range(2), cfg.T, 3000, residual=True)
    n, dt = _oracle_rate(jobs, 1)
    per_layer = dt / 2
    out["glm_verify"] = {"value": cfg.T / (per_layer * cfg.n_layers),
                         "unit": "tokens/s per 8-layer stack", "cores": 1,
                         "s_per_layer": per_layer,
                         "sample": f"T=8 through 2 of the 8 chained layers ({n} token-layers, "
                                   f"{dt:.1f} s), scaled to 8 layers"}
    # Edge0 (T = 1 x 40 chained layers), top-4 and top-8: the whole step
    for name in ("edge0_decode", "edge0_decode_k8"):
        cfg = synth.CONFIGS[name]
        jobs = _oracle_jobs(cfg, range(cfg.n_layers), 1, 4000, residual=True)
        n, dt = _oracle_rate(jobs, 1)
        out[name] = {"value": 1.0 / dt, "unit": "40-layer steps/s (tokens/s)", "cores": 1,
                     "s_per_layer": dt / cfg.n_layers,
                     "sample": f"one token through all {cfg.n_layers} layers ({dt:.2f} s)"}
    # GLM prefill (T = 2048): a 32-token slice, one thread and all cores
    cfg = synth.CONFIGS["glm_prefill"]
    jobs = _oracle_jobs(cfg, [0], 32, 5000)
    n, dt = _oracle_rate(jobs, 1)
    out["glm_prefill"] = {"value": n / dt, "unit": "tokens/s", "cores": 1,
                          "ms_per_2048_layer": 2048 / (n / dt) * 1e3,
                          "sample": f"{n} of the 2048 tokens ({dt:.1f} s), scaled"}
    jobs = _oracle_jobs(cfg, [0], 6 * nproc, 6000)
    n, dt = _oracle_rate(jobs, nproc)
    out["glm_prefill_all_cores"] = {"value": n / dt, "unit": "tokens/s", "cores": nproc,
                                    "ms_per_2048_layer": 2048 / (n / dt) * 1e3,
                                    "sample": f"{n} tokens, {nproc} threads ({dt:.1f} s), scaled"}
    for v in out.values():
        v["kind"] = "oracle"
    return head, out


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-extra", action="store_true", help="only the decode workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=40)
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--only", choices=["decode", "verify", "edge0", "edge0_k8", "prefill", "grouped",
                                       "softmax", "int8_shared", "requant", "staged",
                                       "prefill_int8_shared", "batch"],
                    help="run one workload only (for profiling); the JSON line then "
                         "carries that workload in extra")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this build "
              f"has no multi-GPU path; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    result = {
        "metric": None, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4 x fp16 -> fp32", "data": "synthetic",
        "config": {"workload": "glm_decode: GLM-5.2-shape MoE layer, H=6144, E=256, top-8, "
                               "I=2048, 1 shared expert, int4 per-row scale, T=1, 8 resident "
                               "layers rotated", "global_batch": 1, "seq_len": 1,
                   "parallelism": "none (1 GPU)", "weights": "int4 (fp32 row scales)",
                   "activations": "fp32 in and out; inside the expert GEMVs each 64-input "
                                  "span of x and of h is rounded once to fp16 after an exact "
                                  "power-of-two scale; fp32 accumulate"},
        "extra": {},
    }
    if args.only and args.only != "decode":
        if args.copy_probe:
            copy_probe(torch, result)
        {"verify": lambda: bench_chain(torch, "glm_verify", 64, result),
         "edge0": lambda: bench_chain(torch, "edge0_decode", 200, result),
         "edge0_k8": lambda: bench_chain(torch, "edge0_decode_k8", 200, result),
         "prefill": lambda: bench_prefill(torch, 20, result),
         "prefill_int8_shared": lambda: bench_prefill(torch, 20, result, "glm_prefill_int8_shared"),
         "grouped": lambda: bench_rotated(torch, "glm_decode_grouped", 200, result),
         "softmax": lambda: bench_rotated(torch, "glm_decode_softmax", 200, result),
         "int8_shared": lambda: bench_rotated(torch, "glm_decode_int8_shared", 200, result),
         "batch": lambda: (bench_batch(torch, "glm_batch16", 64, result),
                           bench_batch(torch, "glm_batch32", 64, result)),
         "requant": lambda: bench_requant(torch, result),
         "staged": lambda: bench_staged(torch, result)}[args.only]()
        print(json.dumps(result), flush=True)
        return
    bench_decode(torch, args, result)
    if not args.no_probe:
        ceil = stream_ceiling(torch, result, result["roofline"]["algorithmic_bytes_per_launch"])
        rf = result["roofline"]
        rf["stream_ceiling_gbps"] = ceil
        rf["frac_of_stream_ceiling"] = rf["achieved"] / ceil
        lay = result["extra"]["glm_decode"]
        lay["layer_frac_of_stream_ceiling"] = lay["layer_gbps"] / ceil
    if args.copy_probe:
        copy_probe(torch, result)
    if not args.no_extra and not args.only:
        bench_chain(torch, "glm_verify", 64, result)
        bench_chain(torch, "edge0_decode", 200, result)
        bench_chain(torch, "edge0_decode_k8", 200, result)
        bench_rotated(torch, "glm_decode_grouped", 200, result)
        bench_rotated(torch, "glm_decode_softmax", 200, result)
        bench_rotated(torch, "glm_decode_int8_shared", 200, result)
        bench_batch(torch, "glm_batch16", 64, result)
        bench_batch(torch, "glm_batch32", 64, result)
        bench_requant(torch, result)
        bench_staged(torch, result)
        bench_prefill(torch, 20, result)
        bench_prefill(torch, 10, result, "glm_prefill_int8_shared")
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"], result["extra"]["cpu_baseline_by_workload"] = \
            cpu_baseline(args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
