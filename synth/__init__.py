"""Seeded synthetic inputs for the int4 MoE FFN layer.

Input generation only (see synth.h for the generator's definition): router
weights and bias, expert weights and tokens, on the host (numpy) or in place
in device memory (HIP fill kernel).  Nothing here quantises, routes or
computes any part of the layer, so both the CPU oracle and the GPU library
can consume these inputs without sharing any of the method's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, LayerConfig  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(_HERE, "libsynth_host.so")
GPU_SO = os.path.join(_HERE, "libsynth_gpu.so")

T_ROUTER_W, T_ROUTER_B, T_X, T_GATE, T_UP, T_DOWN, T_PERM = 1, 2, 3, 4, 5, 6, 7

HIPCC_FLAGS = [
    "-O3", "-fPIC", "-shared", "--offload-arch=gfx950", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(gpu: bool = True) -> None:
    """Compile the host fill library (gcc) and the device fill library (hipcc)."""
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
         os.path.join(_HERE, "synth_host.c"), "-o", HOST_SO + ".tmp", "-lm"])
    os.replace(HOST_SO + ".tmp", HOST_SO)
    if gpu:
        subprocess.check_call(
            ["hipcc", *HIPCC_FLAGS, os.path.join(_HERE, "synth_gpu.hip"), "-o", GPU_SO + ".tmp"])
        os.replace(GPU_SO + ".tmp", GPU_SO)


_host = None
_gpu = None


def host_lib() -> ctypes.CDLL:
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            build(gpu=False)
        lib = ctypes.CDLL(HOST_SO)
        u64, u32, f32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p
        lib.synth_fill_gauss.argtypes = [vp, u64, u64, f32, u64]
        lib.synth_fill_gauss.restype = None
        lib.synth_key_c.argtypes = [u64, u32, u32, u32]
        lib.synth_key_c.restype = u64
        lib.synth_u64_c.argtypes = [u64, u64]
        lib.synth_u64_c.restype = u64
        lib.synth_gauss_c.argtypes = [u64, u64, f32]
        lib.synth_gauss_c.restype = f32
        lib.synth_permutation.argtypes = [vp, ctypes.c_int, u64]
        lib.synth_permutation.restype = None
        lib.synth_router_bias.argtypes = [vp, ctypes.c_int, u64, u32, f32, ctypes.c_double,
                                          ctypes.c_double]
        lib.synth_router_bias.restype = None
        _host = lib
    return _host


def gpu_lib() -> ctypes.CDLL:
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_SO):
            raise RuntimeError(f"{GPU_SO} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_SO)
        lib.synth_gpu_fill_gauss.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                             ctypes.c_float, ctypes.c_uint64, ctypes.c_void_p]
        lib.synth_gpu_fill_gauss.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def key(seed: int, layer: int, tensor: int, expert: int = 0) -> int:
    return int(host_lib().synth_key_c(seed, layer, tensor, expert))


def gauss(k: int, n: int, sigma: float, idx0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        host_lib().synth_fill_gauss(out.ctypes.data, n, k, sigma, idx0)
    return out


def permutation(n: int, k: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    host_lib().synth_permutation(out.ctypes.data, n, k)
    return out


def gpu_fill_gauss(ptr: int, n: int, k: int, sigma: float, idx0: int = 0, stream: int = 0) -> None:
    rc = gpu_lib().synth_gpu_fill_gauss(ptr, n, k, sigma, idx0, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_gauss failed ({rc})")


# --------------------------------------------------------------------------
# Per-config tensors.  Shapes follow the layer: router W [E, H], bias [E],
# gate/up [I, H], down [H, I] (row-major, output rows), x [T, H].
# --------------------------------------------------------------------------

def router_weight(cfg: LayerConfig, layer: int) -> np.ndarray:
    k = key(cfg.seed, layer, T_ROUTER_W, 0)
    return gauss(k, cfg.E * cfg.H, cfg.sigma_r).reshape(cfg.E, cfg.H)


def router_bias(cfg: LayerConfig, layer: int) -> np.ndarray:
    out = np.empty(cfg.E, dtype=np.float32)
    host_lib().synth_router_bias(out.ctypes.data, cfg.E, cfg.seed, layer, cfg.sigma_b,
                                 cfg.zipf_c, cfg.zipf_s)
    return out


def expert_keys(cfg: LayerConfig, layer: int, expert: int) -> tuple[int, int, int]:
    """Stream keys of (gate, up, down) of an expert; shared expert s is E + s."""
    return (key(cfg.seed, layer, T_GATE, expert), key(cfg.seed, layer, T_UP, expert),
            key(cfg.seed, layer, T_DOWN, expert))


def expert_weights(cfg: LayerConfig, layer: int, expert: int):
    kg, ku, kd = expert_keys(cfg, layer, expert)
    n = cfg.I * cfg.H
    wg = gauss(kg, n, cfg.sigma_w).reshape(cfg.I, cfg.H)
    wu = gauss(ku, n, cfg.sigma_w).reshape(cfg.I, cfg.H)
    wd = gauss(kd, n, cfg.sigma_w).reshape(cfg.H, cfg.I)
    return wg, wu, wd


def tokens(cfg: LayerConfig, T: int | None = None, stream: int = 0) -> np.ndarray:
    T = cfg.T if T is None else T
    k = key(cfg.seed, 0, T_X, stream)
    return gauss(k, T * cfg.H, cfg.sigma_x).reshape(T, cfg.H)


# --------------------------------------------------------------------------
# Checkpoint-form tensors (inputs of the requantiser): synthetic stand-ins of
# an FP8 E4M3 checkpoint tensor with one fp32 inverse scale per 128 x 128
# block, and of a bf16 one.  Encoding uses torch's casts; nothing here
# decodes or quantises to int4.
# --------------------------------------------------------------------------

def fp8_checkpoint(k: int, O: int, I: int, sigma: float, block: int = 128):
    """codes [O][I] uint8 (E4M3 fn) of N(0, 112) clipped to the format's
    +-448, and inverse scales [ceil(O/B)][ceil(I/B)] fp32 spread
    log-normally (sd 0.3) around sigma * 4 / 448, so that code * scale has
    roughly the spread of N(0, sigma) weights."""
    import torch
    v = np.clip(gauss(k, O * I, 112.0), -448.0, 448.0).reshape(O, I)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nb = ((O + block - 1) // block, (I + block - 1) // block)
    ls = gauss(k, nb[0] * nb[1], 0.3, idx0=O * I).reshape(nb).astype(np.float64)
    sinv = (sigma * 4.0 / 448.0 * np.exp(ls)).astype(np.float32)
    return codes, sinv


def bf16_checkpoint(k: int, O: int, I: int, sigma: float) -> np.ndarray:
    """bf16 bit patterns [O][I] (uint16) of N(0, sigma), rounded by torch."""
    import torch
    w = gauss(k, O * I, sigma).reshape(O, I)
    return torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
