"""Helpers of the GPU parity tests: oracle references for a layer and the
comparison rules.

Comparison rules (the pages fix no MoE output values, so float parity is
against the oracle):
  - expert ids: a token whose K-th and (K+1)-th selection scores are closer
    than 1e-4 (on the oracle's scores) has several correct answers within
    the fp32 router's rounding and is flagged and left out of the id and
    output checks; if only consecutive chosen ranks are that close, the ids
    are compared as a set; otherwise the ordered list must match exactly;
  - outputs: max|gpu - oracle| / max|oracle| <= 2e-3 over unflagged tokens;
  - integer and byte results (packed codes, bucketing): bit-exact.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

TIE_GAP = 1e-4
REL_TOL = 2e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_blob(cfg, layer: int, e: int) -> np.ndarray:
    """Expert e's blob; e >= E is shared expert e - E, in the shared format."""
    fmt = cfg.shared_fmt if (e >= cfg.E and cfg.shared_fmt) else cfg.fmt
    return oracle.pack_expert(fmt, *synth.expert_weights(cfg, layer, e))


def oracle_blobs(cfg, layer: int, experts, workers: int = 8) -> dict:
    experts = sorted(set(int(e) for e in experts))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        blobs = list(ex.map(lambda e: oracle_blob(cfg, layer, e), experts))
    return dict(zip(experts, blobs))


class OracleLayer:
    """Router and only the experts a batch needs, generated on demand."""

    def __init__(self, cfg, layer: int):
        self.cfg, self.layer = cfg, layer
        self.W = synth.router_weight(cfg, layer)
        self.b = synth.router_bias(cfg, layer)
        self.shared = [oracle_blob(cfg, layer, cfg.E + s) for s in range(cfg.n_shared)]
        self.cache: dict = {}

    def route(self, x):
        cfg = self.cfg
        return oracle.route(x, self.W, self.b, cfg.K, cfg.routed_scale, cfg.norm_topk, cfg.n_group,
                            cfg.topk_group, cfg.scoring)

    def need(self, experts):
        missing = [e for e in set(int(v) for v in np.ravel(experts)) if e not in self.cache]
        if missing:
            self.cache.update(oracle_blobs(self.cfg, self.layer, missing))

    def forward(self, x, residual: bool = False, workers: int = 8):
        """out (or x + out for residual), ids, wts, gap_k, gap_in; tokens in
        parallel threads (each oracle call is single-threaded C)."""
        cfg = self.cfg
        x = np.ascontiguousarray(x, dtype=np.float32)
        xin = oracle.rmsnorm(x, cfg.eps) if residual else x
        ids, wts, _, _, gk, gi = self.route(xin)
        self.need(ids)
        blobs = [self.cache.get(e) for e in range(cfg.E)]

        def one(t):
            if residual:
                o, _, _ = oracle.residual_layer(x[t:t + 1], self.W, self.b, cfg.K, cfg.fmt, cfg.I,
                                                blobs, self.shared, cfg.eps, cfg.routed_scale,
                                                cfg.norm_topk, cfg.n_group, cfg.topk_group,
                                                cfg.scoring, cfg.shared_fmt)
            else:
                o, _, _ = oracle.moe_layer(xin[t:t + 1], self.W, self.b, cfg.K, cfg.fmt, cfg.I,
                                           blobs, self.shared, cfg.routed_scale, cfg.norm_topk,
                                           cfg.n_group, cfg.topk_group, cfg.scoring,
                                           cfg.shared_fmt)
            return o[0]

        with ThreadPoolExecutor(max_workers=workers) as ex:
            out = np.stack(list(ex.map(one, range(x.shape[0]))))
        return out, ids, wts, gk, gi


def flags(gk, gi):
    """(excluded, set_compare) boolean masks per token."""
    gk = np.asarray(gk)
    gi = np.asarray(gi)
    excluded = gk < TIE_GAP
    set_cmp = (~excluded) & (gi < TIE_GAP)
    return excluded, set_cmp


def check_ids(ids_gpu, ids_ref, wts_gpu, wts_ref, gk, gi, what=""):
    ids_gpu = np.asarray(ids_gpu)
    excluded, set_cmp = flags(gk, gi)
    n_bad = 0
    for t in range(ids_ref.shape[0]):
        if excluded[t]:
            continue
        if set_cmp[t]:
            ok = set(ids_gpu[t].tolist()) == set(ids_ref[t].tolist())
            if ok:
                mg = dict(zip(ids_gpu[t].tolist(), np.asarray(wts_gpu)[t].tolist()))
                mr = dict(zip(ids_ref[t].tolist(), wts_ref[t].tolist()))
                ok = all(abs(mg[e] - mr[e]) <= 1e-5 * max(1.0, abs(mr[e])) for e in mr)
        else:
            ok = np.array_equal(ids_gpu[t], ids_ref[t]) and np.allclose(
                np.asarray(wts_gpu)[t], wts_ref[t], rtol=1e-5, atol=1e-6)
        if not ok:
            n_bad += 1
            log(f"{what} token {t}: ids gpu {ids_gpu[t]} ref {ids_ref[t]} "
                f"w gpu {np.asarray(wts_gpu)[t]} ref {wts_ref[t]} gap_k {gk[t]:.3g}")
    assert n_bad == 0, f"{what}: {n_bad} tokens with mismatched routing"
    return int(excluded.sum())


def rel_err(out_gpu, out_ref, keep=None) -> float:
    og = np.asarray(out_gpu, dtype=np.float64)
    orf = np.asarray(out_ref, dtype=np.float64)
    if keep is not None:
        og, orf = og[keep], orf[keep]
    if orf.size == 0:
        return 0.0
    return float(np.abs(og - orf).max() / max(np.abs(orf).max(), 1e-30))


def check_residual(x, got_next, ref_next, keep=None, what=""):
    """A residual step x <- x + moe(rmsnorm(x)) checked twice at REL_TOL:
    the new x, and the MoE term alone (got_next - x against ref_next - x),
    so that a large x cannot hide an error in the term.  Returns both
    relative errors."""
    x = np.asarray(x, dtype=np.float64)
    e_next = rel_err(got_next, ref_next, keep)
    e_term = rel_err(np.asarray(got_next, dtype=np.float64) - x,
                     np.asarray(ref_next, dtype=np.float64) - x, keep)
    assert e_next <= REL_TOL, f"{what}: new x max|d|/max|ref| = {e_next:.3e}"
    assert e_term <= REL_TOL, f"{what}: moe term max|d|/max|ref| = {e_term:.3e}"
    return e_next, e_term


WORKERS = min(16, os.cpu_count() or 1)


def block_sample(ids, E, excluded, block=32):
    """Tokens that put a compared row in every occupied 32-row block of the
    grouped GEMM: an expert's rows are its tokens in ascending order (the
    stable bucketing), the shared expert's rows are all tokens.  Each block
    contributes its last unflagged token; a block of near-tie tokens only
    (a rarely chosen expert whose few tokens all sit on a tie, where either
    side may route differently) is left out and counted."""
    T, _ = ids.shape
    picks, uncovered = set(), 0
    groups = [np.flatnonzero((ids == e).any(axis=1)) for e in range(E)] + [np.arange(T)]
    for toks in groups:
        for b0 in range(0, len(toks), block):
            blk = toks[b0:b0 + block]
            ok = blk[~excluded[blk]]
            if len(ok):
                picks.add(int(ok[-1]))
            else:
                uncovered += 1
    return np.array(sorted(picks)), uncovered
