"""Seeded synthetic inputs for the BitLinear forward.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
bench.  It draws random numbers only; it contains none of the method's
arithmetic (no scales, no rounding to codes, no packing, no contraction).

Generator
---------
SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; the finaliser constants are the ones of Vigna's public
splitmix64.c), used as a counter-based generator: draw ``i`` of stream ``key``
is ``mix(key + (i + 1) * 0x9E3779B97F4A7C15)``.  Uniforms take the top 53 bits;
normals use the cosine branch of Box-Muller in float64 (one normal per two
uniforms).  Everything is expressed in torch int64 / float64 ops so it runs on
the CPU or on a GPU; the integer stream is bit-identical on both devices, the
float64 transcendental step may differ in its last bit between devices, which is
why every parity check compares results computed from the very bytes that were
handed to the GPU.

Workload recipes (the pages give the model shapes only in prose; these follow
the configurations the bench and tests exercise):

* activations: bf16 ~ N(0, 1), optionally with ``round(0.001 * M * K)``
  positions (chosen uniformly without replacement) scaled by 20 (outliers), or
  with a per-row scale drawn from U[0.1, 10];
* latent weights: fp32 ~ N(0, sigma) with sigma 0.02 (2.4B-model shapes) or 0.01
  (100B-scale shapes);
* density-controlled latent weights: code t with P(0) = 1 - d, P(+-1) = d / 2,
  latent w = 0.02 * t.
"""
from __future__ import annotations

import math

import torch

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Two's-complement view of an unsigned 64-bit constant as a signed int64."""
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 lanes holding unsigned 64-bit values."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _s64(_M1)
    z = (z ^ _srl(z, 27)) * _s64(_M2)
    return z ^ _srl(z, 31)


def mix64_py(v: int) -> int:
    """Pure-Python SplitMix64 finaliser (used to derive stream keys)."""
    z = v & _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def splitmix64_py(key: int, n: int) -> list[int]:
    """Reference draws 0..n-1 of stream ``key`` in plain Python integers."""
    return [mix64_py(key + (i + 1) * _GAMMA) for i in range(n)]


def stream_key(*parts: int) -> int:
    """Derive a 64-bit stream key from integers such as (config, seed, tensor)."""
    k = 0x243F6A8885A308D3
    for p in parts:
        k = mix64_py(k ^ (p & _MASK64))
    return k


def raw64(key: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Draws start..start+count-1 of stream ``key`` as int64 lanes."""
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    z = i * _s64(_GAMMA) + _s64(key)
    return _mix(z)


def uniform(key: int, count: int, start: int = 0, device="cpu") -> torch.Tensor:
    """float64 uniforms in [0, 1) from the top 53 bits of each draw."""
    return _srl(raw64(key, start, count, device), 11).to(torch.float64) * (2.0 ** -53)


def normal(key: int, count: int, device="cpu", chunk: int = 1 << 26) -> torch.Tensor:
    """float64 N(0, 1) by Box-Muller (cosine branch), draws 2i and 2i+1 -> normal i."""
    out = torch.empty(count, dtype=torch.float64, device=device)
    for s in range(0, count, chunk):
        n = min(chunk, count - s)
        u = uniform(key, 2 * n, 2 * s, device).view(n, 2)
        r = torch.sqrt(-2.0 * torch.log1p(-u[:, 0]))
        out[s:s + n] = r * torch.cos((2.0 * math.pi) * u[:, 1])
    return out


def latent_weights(key: int, N: int, K: int, sigma: float, device="cpu") -> torch.Tensor:
    """fp32 [N][K] latent weights ~ N(0, sigma)."""
    out = torch.empty(N * K, dtype=torch.float32, device=device)
    chunk = 1 << 25
    for s in range(0, N * K, chunk):
        n = min(chunk, N * K - s)
        sub = stream_key(key, s)
        out[s:s + n] = (normal(sub, n, device) * sigma).to(torch.float32)
    return out.view(N, K)


def density_weights(key: int, N: int, K: int, density: float, device="cpu") -> torch.Tensor:
    """fp32 [N][K] latent weights 0.02 * t with t in {-1, 0, +1}, P(t != 0) = density."""
    u = uniform(key, N * K, 0, device)
    t = torch.zeros(N * K, dtype=torch.float32, device=device)
    t[u < density / 2] = -1.0
    t[(u >= density / 2) & (u < density)] = 1.0
    return (t * 0.02).view(N, K)


def activations(key: int, M: int, K: int, outlier_frac: float = 0.0,
                row_scale: tuple[float, float] | None = None, device="cpu") -> torch.Tensor:
    """bf16 [M][K] activations ~ N(0, 1).

    outlier_frac: exactly round(outlier_frac * M * K) distinct positions, picked
    as the smallest keys of an independent uniform stream, are multiplied by 20.
    row_scale: (lo, hi) -> every row is multiplied by its own U[lo, hi] draw.
    Scaling happens in fp32; the result is rounded to bf16 (round to nearest even).
    """
    x = normal(stream_key(key, 1), M * K, device).to(torch.float32)
    n_out = int(round(outlier_frac * M * K))
    if n_out > 0:
        u = uniform(stream_key(key, 2), M * K, 0, device)
        idx = torch.topk(u, n_out, largest=False).indices
        x[idx] = x[idx] * 20.0
    x = x.view(M, K)
    if row_scale is not None:
        lo, hi = row_scale
        s = (lo + (hi - lo) * uniform(stream_key(key, 3), M, 0, device)).to(torch.float32)
        x = x * s[:, None]
    return x.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Raw bf16 bit patterns as uint16-compatible int16 view."""
    assert x.dtype == torch.bfloat16
    return x.view(torch.int16)


def random_bytes(key: int, count: int, device="cpu") -> torch.Tensor:
    """count uniformly random bytes (every 2-bit field may be 0..3)."""
    return (_srl(raw64(key, 0, count, device), 56)).to(torch.uint8)
