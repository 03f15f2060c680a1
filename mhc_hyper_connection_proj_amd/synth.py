"""Seeded synthetic inputs for the mHC path.

This module only draws random numbers and stores them in their storage type.
It contains none of the method's arithmetic, so the parity tests can feed the
same host arrays to the HIP library and to the CPU oracle.

Seeding: numpy PCG64 with seed = 1000 * workload_id + tensor_id, where the
tensor ids are X=1, W=2, x=3, bias=4, G=5, H_res logits=6, H_post logits=7,
layer scale=8, norm gain=9, norm upstream grad=10.  Normals are drawn in float32 and scaled by their standard
deviation; bf16 tensors are the round-to-nearest-even bf16 of those float32
values, returned as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TENSOR_IDS = {"X": 1, "W": 2, "x": 3, "bias": 4, "G": 5, "L": 6, "Hpost_logits": 7, "scale": 8, "gamma": 9,
              "dy": 10}


@dataclass(frozen=True)
class Workload:
    """Shapes and distributions of one synthetic workload."""
    wid: int
    name: str
    tokens: int          # B*T
    n: int
    C: int
    act: str             # storage type of residual-shaped activations: 'bf16' or 'f32'
    iters: int = 20
    eps: float = 1e-6
    rms_eps: float = 1e-6
    w_std: float = 0.02
    bias_std: float = 0.1
    has_bias: bool = True
    description: str = ""


WORKLOADS = {
    "tiny_chain": Workload(
        1, "tiny_chain", tokens=64, n=4, C=256, act="f32",
        description="B=1,T=64,n=4,C=256; fp32 residual N(0,1); W N(0,0.02) [1024,24]; "
                    "x N(0,1) [64,256]; bias N(0,0.1) [256]; 20 Sinkhorn iters, eps=1e-6"),
    "sinkhorn_batched": Workload(
        2, "sinkhorn_batched", tokens=256 * 4096, n=4, C=0, act="f32", has_bias=False,
        description="1,048,576 independent 4x4 fp32 logit matrices N(0,1), 20 iters, eps=1e-6, "
                    "upstream grad N(0,1)"),
    "pre_fwd": Workload(
        3, "pre_fwd", tokens=8 * 4096, n=4, C=4096, act="bf16", has_bias=False,
        description="bf16 residual [8,4096,4,4096] N(0,1); fp32 W [16384,24] N(0,0.02)"),
    "post_bda": Workload(
        4, "post_bda", tokens=8 * 4096, n=4, C=4096, act="bf16",
        description="bf16 residual/x/G N(0,1), bf16 bias N(0,0.1) [4096]; H_res = 20-iter "
                    "Sinkhorn of N(0,1) logits; H_post = 2*sigmoid(N(0,1))"),
    "full_layer": Workload(
        5, "full_layer", tokens=4 * 4096, n=4, C=7168, act="bf16", has_bias=False,
        description="B=4,T=4096,n=4,C=7168 bf16 residual N(0,1); fp32 W [28672,24] N(0,0.02); "
                    "layer = per-channel bf16 scale U(0.5,1.5); no bias; upstream grad N(0,1)"),
}


def rng(wid: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * wid + TENSOR_IDS[tensor]))


def normal_f32(wid: int, tensor: str, shape, std: float = 1.0) -> np.ndarray:
    a = rng(wid, tensor).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def uniform_f32(wid: int, tensor: str, shape, lo: float, hi: float) -> np.ndarray:
    a = rng(wid, tensor).random(size=shape, dtype=np.float32)
    return (a * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(a_f32: np.ndarray, act: str) -> np.ndarray:
    """Put float32 draws into the activation storage type (bf16 bits or float32)."""
    return f32_to_bf16_bits(a_f32) if act == "bf16" else np.ascontiguousarray(a_f32, np.float32)


def tensor(w: Workload, name: str, tokens: int | None = None, C: int | None = None) -> np.ndarray:
    """One named input of a workload, optionally at a reduced token count / width.

    Names: X [N,n,C] (act), W [n*C, n*n+2n] f32, x [N,C] (act), bias [C] (act),
    G [N,n,C] (act), L [N,n,n] f32 (logits), Hpost_logits [N,n] f32,
    scale [C] (act, U(0.5,1.5)), dH [N,n,n] f32 (Sinkhorn upstream grad),
    gamma [C] f32 U(0.5,1.5) (norm gain), dy [N,C] (act, N(0,1): upstream grad of the norm).
    """
    N = w.tokens if tokens is None else tokens
    C = w.C if C is None else C
    n = w.n
    if name == "X":
        return store(normal_f32(w.wid, "X", (N, n, C)), w.act)
    if name == "W":
        return normal_f32(w.wid, "W", (n * C, n * n + 2 * n), w.w_std)
    if name == "x":
        return store(normal_f32(w.wid, "x", (N, C)), w.act)
    if name == "bias":
        return store(normal_f32(w.wid, "bias", (C,), w.bias_std), w.act)
    if name == "G":
        return store(normal_f32(w.wid, "G", (N, n, C)), w.act)
    if name == "L":
        return normal_f32(w.wid, "L", (N, n, n))
    if name == "dH":
        return normal_f32(w.wid, "G", (N, n, n))
    if name == "Hpost_logits":
        return normal_f32(w.wid, "Hpost_logits", (N, n))
    if name == "gamma":
        return uniform_f32(w.wid, "gamma", (C,), 0.5, 1.5)
    if name == "dy":
        return store(normal_f32(w.wid, "dy", (N, C)), w.act)
    if name == "scale":
        return store(uniform_f32(w.wid, "scale", (C,), 0.5, 1.5), w.act)
    raise KeyError(name)
