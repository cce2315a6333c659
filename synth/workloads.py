"""Shapes and seeds of the workloads the tests and the bench run.

No arithmetic of the method lives here: only which matrices exist, their
shapes (K = in_features, N = out_features), and which random stream feeds each
tensor.  Pages: chenxutan.com sec. 3.1 (every linear of a standard Transformer
block -- q, k, v, o projections and the gate / up / down FFN -- becomes a
BitLinear); okforks.com sec. 03 (the official ~2.4B-parameter model).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import activations, density_weights, latent_weights, stream_key

# 2.4B-shaped transformer layer: hidden 2560, kv width 640, FFN 6912.
LAYER_2P4B = (("q", 2560, 2560), ("k", 2560, 640), ("v", 2560, 640), ("o", 2560, 2560),
              ("gate", 2560, 6912), ("up", 2560, 6912), ("down", 6912, 2560))
# activation slot per matrix: q/k/v share the attention input, o reads the
# attention output, gate/up share the FFN input, down reads the FFN hidden state
SLOT_2P4B = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
SLOT_K_2P4B = (2560, 2560, 2560, 6912)

# 100B-scale FFN: hidden 8192, FFN 28672.
FFN_100B = (("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192))

CFG_SINGLE, CFG_DECODE, CFG_SWEEP, CFG_PREFILL, CFG_FFN100B = range(5)


@dataclass(frozen=True)
class Matrix:
    layer: int
    name: str
    K: int
    N: int
    sigma: float
    key: int
    slot: int = 0


def decode_step_2p4b(layers: int = 30):
    """The 7 x layers matrices of one decode step; seed = layer index."""
    out = []
    for l in range(layers):
        for i, (name, K, N) in enumerate(LAYER_2P4B):
            out.append(Matrix(l, name, K, N, 0.02, stream_key(CFG_DECODE, l, i), SLOT_2P4B[name]))
    return out


def decode_step_activations(layer: int, device="cpu", M: int = 1):
    """The 4 bf16 [M][K] activations of one layer (no outliers); M > 1 is a batch of
    M sequences decoding together."""
    return [activations(stream_key(CFG_DECODE, layer, 100 + s, *((M,) if M > 1 else ())), M, K, device=device)
            for s, K in enumerate(SLOT_K_2P4B)]


# activation slots that an RMSNorm precedes (the attention input and the FFN input
# of chenxutan.com sec. 3.1's block); the other two read the attention output and
# the FFN hidden state
NORMED_SLOTS_2P4B = (0, 2)


def decode_step_gains(layer: int, device="cpu"):
    """fp32 RMSNorm gains of one layer, {slot: [K]}: 1 + 0.1 N(0, 1), seeded per
    layer and slot (random-init stand-ins for the trained gains)."""
    from . import normal
    out = {}
    for s in NORMED_SLOTS_2P4B:
        K = SLOT_K_2P4B[s]
        g = 1.0 + 0.1 * normal(stream_key(CFG_DECODE, layer, 200 + s), K, device).to(torch.float64)
        out[s] = g.to(torch.float32)
    return out


# activation slot whose row is the SwiGLU output, fp32 (the down projection's input
# in chenxutan.com sec. 3.1's block)
SWIGLU_SLOT_2P4B = 3


def decode_step_ffn_hidden(layer: int, device="cpu"):
    """fp32 [1][6912] row of one layer standing in for the SwiGLU output that feeds
    the down projection: N(0, 1), seeded per layer (synthetic)."""
    from . import normal
    K = SLOT_K_2P4B[SWIGLU_SLOT_2P4B]
    return normal(stream_key(CFG_DECODE, layer, 300), K, device).to(torch.float32).reshape(1, K).contiguous()


def ffn_100b(layers: int = 8):
    out = []
    for l in range(layers):
        for i, (name, K, N) in enumerate(FFN_100B):
            out.append(Matrix(l, name, K, N, 0.01, stream_key(CFG_FFN100B, l, i), 0 if name != "down" else 1))
    return out


def ffn_100b_activations(layer: int, M: int, device="cpu"):
    return [activations(stream_key(CFG_FFN100B, layer, 100 + s, M), M, K, device=device)
            for s, K in enumerate((8192, 28672))]


def weights(mat: Matrix, device="cpu") -> torch.Tensor:
    """fp32 [N][K] latent weights of a matrix."""
    return latent_weights(mat.key, mat.N, mat.K, mat.sigma, device)


def single_gemv(device="cpu"):
    """M = 1, K = N = 2560, 0.1% x20 outliers, seed 0."""
    x = activations(stream_key(CFG_SINGLE, 0, 1), 1, 2560, outlier_frac=0.001, device=device)
    w = latent_weights(stream_key(CFG_SINGLE, 0, 2), 2560, 2560, 0.02, device)
    return x, w


def sweep_activations(M: int, device="cpu"):
    """K = 2560, M tokens, 0.1% x20 outliers, seed 0."""
    return activations(stream_key(CFG_SWEEP, 0, M), M, 2560, outlier_frac=0.001, device=device)


def sweep_weights(device="cpu"):
    """The FFN up shape K = 2560, N = 6912, N(0, 0.02) latent weights, seed 0."""
    return latent_weights(stream_key(CFG_SWEEP, 0, 99), 6912, 2560, 0.02, device)


PREFILL_SHAPES = (("up", 2560, 6912), ("down", 6912, 2560))


def prefill_inputs(name: str, density: float | None = None, device="cpu"):
    """M = 2048 tokens, per-row scale U[0.1, 10]; density None = N(0, 0.02) latent
    weights, else codes with P(nonzero) = density."""
    K, N = {n: (k, nn) for n, k, nn in PREFILL_SHAPES}[name]
    idx = 0 if name == "up" else 1
    x = activations(stream_key(CFG_PREFILL, 0, idx), 2048, K, row_scale=(0.1, 10.0), device=device)
    if density is None:
        w = latent_weights(stream_key(CFG_PREFILL, 0, 10 + idx), N, K, 0.02, device)
    else:
        w = density_weights(stream_key(CFG_PREFILL, 0, 20 + idx, int(density * 100)), N, K, density, device)
    return x, w
