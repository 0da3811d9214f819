"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no quantization or GEMM arithmetic: it only draws random
numbers and rounds them to the input dtype (the BF16 rounding is torch's own
cast).  Both the HIP path's tests/benchmark and the oracle's tests take their
inputs from here, so both sides see identical bytes.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: output i of a stream is
mix64(state0 + (i + 1) * 0x9E3779B97F4A7C15), so any slice can be produced
independently and in parallel.  Uniforms are ((z >> 11) + 0.5) * 2^-53 in
(0, 1); normals come from the Box-Muller transform (both the cosine and the
sine branch); Student-t(3) is Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3).

Workloads (N(0, v) names the *variance* v):

* ``tiny_linear``   x BF16 [512,128] N(0,1) (B=8, T=64, D=128); W BF16
  [128,128] N(0,1/128); bias FP32 [128] N(0,0.01).
* ``rowwise_int8``  a FP32 [128,1024] N(0,1); b FP32 [512,1024] N(0,1).
* ``mlp_up``        x BF16 [2048,1024] N(0,1) with 10 seeded columns (1%)
  scaled x20 before rounding; W BF16 [4096,1024] N(0,1/1024); bias FP32
  [4096] N(0,0.01).
* ``mlp_backward``  G BF16 [2048,4096] N(0,1e-3) with ``mlp_up``'s x and W.
* ``large_fp8``     a BF16 [16384,8192] Student-t(3); b BF16 [8192,8192]
  N(0,1/8192).
* ``per_head``      q, k FP32 [16,196,64] N(0,1) (BH=16, N=196, D=64);
  for the softmax.V product (N != M): p FP32 [16,196,160] U(0, 2/160)
  (non-negative, mean 1/160 like attention weights over 160 keys) and
  v FP32 [16,160,64] N(0,1) with head h scaled by 2^(h mod 4 - 1), so the
  heads' ranges differ.

Seeds are 0x5EED0000 + workload number (1..5); each tensor has its own
stream id.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

WORKLOAD_IDS = {"tiny_linear": 1, "rowwise_int8": 2, "mlp_up": 3, "mlp_backward": 4, "large_fp8": 5,
                "per_head": 6}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def splitmix64(state0: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream from state0."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(state0 & 0xFFFFFFFFFFFFFFFF) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _state0(seed: int, stream: int) -> int:
    return ((seed & 0xFFFFFFFF) << 16) | (stream & 0xFFFF)


def uniform(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    z = splitmix64(_state0(seed, stream), start, count)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def _normal_chunk(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Normals start .. start+count-1 (start even); pairs share one draw."""
    p0 = start // 2
    npairs = (count + 1) // 2
    u = uniform(seed, stream, 2 * p0, 2 * npairs).reshape(npairs, 2)
    r = np.sqrt(-2.0 * np.log(u[:, 0]))
    t = 2.0 * math.pi * u[:, 1]
    out = np.empty((npairs, 2), dtype=np.float64)
    out[:, 0] = r * np.cos(t)
    out[:, 1] = r * np.sin(t)
    return out.reshape(-1)[:count]


def _parallel(fn, n: int, chunk: int = _CHUNK) -> np.ndarray:
    """fn(start, count) -> float32 array, evaluated in chunks on a pool."""
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, chunk))

    def work(s):
        c = min(chunk, n - s)
        out[s:s + c] = fn(s, c)

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(_threads()) as pool:
            list(pool.map(work, starts))
    return out


def normal(seed: int, stream: int, n: int, std: float = 1.0) -> np.ndarray:
    """n float32 draws of N(0, std^2)."""
    return _parallel(lambda s, c: (std * _normal_chunk(seed, stream, s, c)).astype(np.float32), n)


def student_t3(seed: int, stream: int, n: int) -> np.ndarray:
    """n float32 draws of Student-t with 3 degrees of freedom."""
    def fn(s, c):
        z = _normal_chunk(seed, stream, 4 * s, 4 * c).reshape(c, 4)
        chi2 = z[:, 1] ** 2 + z[:, 2] ** 2 + z[:, 3] ** 2
        return (z[:, 0] / np.sqrt(chi2 / 3.0)).astype(np.float32)
    return _parallel(fn, n, _CHUNK // 4)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A seeded permutation of range(n) (argsort of uniforms)."""
    return np.argsort(uniform(seed, stream, 0, n), kind="stable")


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """Round float32 to BF16 (torch's round-to-nearest-even cast)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (the oracle's BF16 input)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _seed(workload: str) -> int:
    return 0x5EED0000 + WORKLOAD_IDS[workload]


def workload(name: str) -> dict:
    """CPU tensors of one workload, keyed by role."""
    s = _seed(name)
    if name == "tiny_linear":
        return dict(
            x=to_bf16(normal(s, 0, 512 * 128).reshape(512, 128)),
            w=to_bf16(normal(s, 1, 128 * 128, math.sqrt(1.0 / 128)).reshape(128, 128)),
            bias=torch.from_numpy(normal(s, 2, 128, 0.1)),
        )
    if name == "rowwise_int8":
        return dict(
            a=torch.from_numpy(normal(s, 0, 128 * 1024).reshape(128, 1024)),
            b=torch.from_numpy(normal(s, 1, 512 * 1024).reshape(512, 1024)),
        )
    if name == "mlp_up":
        x = normal(s, 0, 2048 * 1024).reshape(2048, 1024)
        cols = permutation(s, 3, 1024)[:10]
        x[:, cols] *= np.float32(20.0)
        return dict(
            x=to_bf16(x),
            w=to_bf16(normal(s, 1, 4096 * 1024, math.sqrt(1.0 / 1024)).reshape(4096, 1024)),
            bias=torch.from_numpy(normal(s, 2, 4096, 0.1)),
            outlier_cols=torch.from_numpy(np.sort(cols)),
        )
    if name == "mlp_backward":
        up = workload("mlp_up")
        return dict(
            g=to_bf16(normal(s, 0, 2048 * 4096, math.sqrt(1e-3)).reshape(2048, 4096)),
            x=up["x"], w=up["w"],
        )
    if name == "large_fp8":
        return dict(
            a=to_bf16(student_t3(s, 0, 16384 * 8192).reshape(16384, 8192)),
            b=to_bf16(normal(s, 1, 8192 * 8192, math.sqrt(1.0 / 8192)).reshape(8192, 8192)),
        )
    if name == "per_head":
        bh, n, nk, d = 16, 196, 160, 64
        v = normal(s, 3, bh * nk * d).reshape(bh, nk, d)
        v *= (np.float32(2.0) ** (np.arange(bh) % 4 - 1).astype(np.float32))[:, None, None]
        return dict(
            q=torch.from_numpy(normal(s, 0, bh * n * d).reshape(bh, n, d)),
            k=torch.from_numpy(normal(s, 1, bh * n * d).reshape(bh, n, d)),
            p=torch.from_numpy((uniform(s, 2, 0, bh * n * nk) * (2.0 / nk)).astype(np.float32).reshape(bh, n, nk)),
            v=torch.from_numpy(v),
        )
    raise KeyError(name)


def random_bf16(seed: int, stream: int, rows: int, cols: int, std: float = 1.0) -> torch.Tensor:
    """A BF16 [rows, cols] N(0, std^2) matrix for tests of arbitrary shape."""
    return to_bf16(normal(seed, stream, rows * cols, std).reshape(rows, cols))


def random_fp32(seed: int, stream: int, rows: int, cols: int, std: float = 1.0) -> torch.Tensor:
    return torch.from_numpy(normal(seed, stream, rows * cols, std).reshape(rows, cols))


def random_codes(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """Uniform random bytes [rows, cols] (callers mask out NaN/inf codes)."""
    z = splitmix64(_state0(seed, stream), 0, rows * cols)
    return (z >> np.uint64(56)).astype(np.uint8).reshape(rows, cols)
